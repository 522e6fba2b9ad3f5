// evict.hip -- eviction on a KIVI-style 4-bit cache: the kept tokens of every (b, h) form a
// new cache of K tokens whose last R2 stay bf16.
//
// Explainer (KV cache 压缩：把历史装得更小), eviction section (only the selected KV stays)
// applied to the 4-bit layout of its grouping-axis and residual-budget sections; the
// Walkthrough (KV Compression 公式到源码对照) §4 multiplies the token saving with the byte
// saving.  What happens to a group:
//   - V groups lie inside one token, so a kept quantized V row keeps its codes, scale, zero;
//   - a K group spans g tokens of one channel.  A new K group whose tokens are exactly one
//     whole old group, in order, keeps that group's codes, scale and zero; any other new K
//     group is quantized afresh, per channel, from the current values of its tokens (the
//     dequantized levels, exact in fp32, or the bf16 window values);
//   - a window token that lands in the quantized part is quantized like a new token;
//   - a new window row holds the current value rounded to the nearest bf16.
//
// One launch, two kinds of block, each over one (b, h) (block order (b, tile, h), h fastest):
//   group blocks: the g new quantized tokens of one new K group, K and V.  The keep indices go
//     to LDS; one block-wide vote decides "whole old group".  Every lane owns 8 channels of
//     RPP-strided rows and issues the loads of all its rows before using any (the 4-bit rows
//     unconditionally, from the clamped row, so no load waits behind a branch).  V rows are
//     copied or, for window tokens, quantized (the g-channel groups reduce across g/8 lanes
//     with shuffles).  K is copied when whole, else the rows are dequantized in registers and
//     the group's min/max, parameters and codes follow the quantizer's steps.
//   window blocks: 64 new bf16 rows; copy, or dequantize and round to bf16.
// Keep indices outside [0, T) are clamped into it: the result is then unspecified, but no
// access leaves the source sections.
#include "int4_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;   // rows per V / window block

struct EvGeom {
    int64_t T, H, Tq;                 // source tokens, heads, quantized tokens
    int64_t ldq, ldk, ldr;            // source rows per (b, h): codes / V params, K params, window
    int64_t K, Tq2, R2;               // kept tokens, of which quantized / window
    int64_t dldq, dldk, dldr;         // destination rows per (b, h)
    int64_t nKb, nRb;                 // blocks per (b, h) of each kind
};

__device__ __forceinline__ int64_t clamp_tok(int32_t t, int64_t T) {
    return t < 0 ? 0 : (t >= T ? T - 1 : (int64_t)t);
}

// 8 codes of one packed dword (low nibble = even channel) as floats.
__device__ __forceinline__ void unpack_codes8(uint32_t w, float (&c)[8]) {
    const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c[2 * e] = (float)((lo >> (8 * e)) & 0xffu);
        c[2 * e + 1] = (float)((hi >> (8 * e)) & 0xffu);
    }
}

// Raw source data of one kept token for one lane (8 channels), loaded without a branch: the
// codes and the V scale/zero from the quantized row min(t, Tq - 1) (unused for a window
// token), and two 16-byte words whose address depends on the token: the K group scale and
// zero rows for a quantized token, its bf16 K and V rows for a window token.
struct RowRaw {
    uint32_t kc, vc;
    uint4 a, b;        // quantized: K scale, K zero;  window: K row, V row
    uint16_t vs, vz;
};

template <int D, int G>
__device__ __forceinline__ void load_row(const kvq_int4_cache& s, const EvGeom& geo, int64_t bh, int64_t t, int lane,
                                         RowRaw& r) {
    const bool q = t < geo.Tq;
    if (geo.Tq > 0) {   // uniform: with no quantized tokens the 4-bit sections may be empty
        const int64_t tq = q ? t : geo.Tq - 1;
        r.kc = *reinterpret_cast<const uint32_t*>(s.k_codes + (bh * geo.ldq + tq) * (D / 2) + 4 * lane);
        r.vc = *reinterpret_cast<const uint32_t*>(s.v_codes + (bh * geo.ldq + tq) * (D / 2) + 4 * lane);
        const int64_t mv = (bh * geo.ldq + tq) * (D / G) + (8 * lane) / G;
        r.vs = s.v_scale[mv];
        r.vz = s.v_zero[mv];
    }
    const int64_t mk = (bh * geo.ldk + (q ? t / G : 0)) * D + 8 * lane;         // quantized token
    const int64_t mr = (bh * geo.ldr + (q ? 0 : t - geo.Tq)) * D + 8 * lane;    // window token
    const uint16_t* pa = q ? s.k_scale + mk : s.k_res + mr;
    const uint16_t* pb = q ? s.k_zero + mk : s.v_res + mr;
    r.a = *reinterpret_cast<const uint4*>(pa);
    r.b = *reinterpret_cast<const uint4*>(pb);
}

// Current values (fp32) of the lane's 8 channels: (q - z) * s rounded once (q*s and z*s are
// exact in fp32, so the fma rounds the exact value once), or the bf16 window values.
__device__ __forceinline__ void k_values(const RowRaw& r, bool quantized, float (&v)[8]) {
    if (quantized) {
        float sc[8], zf[8], c[8];
        unpack8(r.a, sc);
        unpack8(r.b, zf);
        unpack_codes8(r.kc, c);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(c[k], sc[k], -zf[k] * sc[k]);
    } else {
        unpack8(r.a, v);
    }
}

__device__ __forceinline__ void v_values(const RowRaw& r, bool quantized, float (&v)[8]) {
    if (quantized) {
        const float sc = bf_to_f(r.vs), zs = -bf_to_f(r.vz) * sc;
        float c[8];
        unpack_codes8(r.vc, c);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(c[k], sc, zs);
    } else {
        unpack8(r.b, v);
    }
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads) int4_evict_kernel(const kvq_int4_cache src, const int32_t* __restrict__ keep,
                                                              kvq_int4_cache dst, EvGeom geo) {
    constexpr int LPR = D / 8;            // lanes per token row (8 channels each)
    constexpr int RPP = kThreads / LPR;   // rows per pass
    constexpr int NW = kThreads / 64;
    constexpr int NGD = D / G;
    constexpr int LPG = G / 8;            // lanes per V group
    const int tid = threadIdx.x, lane = tid % LPR, rg = tid / LPR, wave = tid / 64;
    const uint32_t H = (uint32_t)geo.H;
    uint32_t bid = blockIdx.x;
    const uint32_t nK = (uint32_t)(src.B * geo.nKb * geo.H);

    if (bid < nK) {
        // ------------- one new K group and the V rows of the same G tokens -------------
        static_assert(G % RPP == 0, "tile shape");
        constexpr int NR = G / RPP;
        __shared__ float s_mn[NW * D], s_mx[NW * D];
        __shared__ float s_ps[D], s_pr[D], s_pz[D];
        const Bjh ix = split_bjh(bid, H, (uint32_t)geo.nKb);
        const int64_t bh = ix.b * geo.H + ix.h, j = ix.j, i0 = j * G;
        const int n = (int)min<int64_t>(G, geo.Tq2 - i0);
        const int32_t* kp = keep + bh * geo.K + i0;
        const int64_t first = clamp_tok(kp[0], geo.T);
        // this thread's rows (rows past the group repeat row 0), then all of their loads; the
        // block-wide "whole old group" vote waits until the loads are in flight
        RowRaw raw[NR];
        int64_t tok[NR];
        int run = 1;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = rg + RPP * i;
            tok[i] = clamp_tok(kp[r < n ? r : 0], geo.T);
            run &= (r >= n) || (tok[i] == first + r);
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) load_row<D, G>(src, geo, bh, tok[i], lane, raw[i]);
        const bool whole = __syncthreads_and(run) && first < geo.Tq && first % G == 0 &&
                           n == (int)min<int64_t>(G, geo.Tq - first);

        // V rows: a quantized row keeps codes, scale and zero; a window row is quantized.  The
        // group reduction runs for every row (the G/8 lanes of a group share the row, so the
        // shuffles never cross rows), the result is used for window rows only.
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = rg + RPP * i;
            const bool q = tok[i] < geo.Tq;
            float x[8];
            v_values(raw[i], q, x);
            float mn = FLT_MAX, mx = -FLT_MAX;
            minmax8(x, mn, mx);
            mn = lane_group_reduce<LPG, false>(mn);
            mx = lane_group_reduce<LPG, true>(mx);
            if (r < n) {
                uint8_t* crow = dst.v_codes + (bh * geo.dldq + i0 + r) * (D / 2);
                const int64_t dmi = (bh * geo.dldq + i0 + r) * NGD + (8 * lane) / G;
                if (q) {
                    *reinterpret_cast<uint32_t*>(crow + 4 * lane) = raw[i].vc;
                    if (lane % LPG == 0) {
                        dst.v_scale[dmi] = raw[i].vs;
                        dst.v_zero[dmi] = raw[i].vz;
                    }
                } else {
                    const GroupParams gp = group_params(mn, mx);
                    if (lane % LPG == 0) {
                        dst.v_scale[dmi] = gp.sb;
                        dst.v_zero[dmi] = gp.zb;
                    }
                    const bool fast = gp.z >= 0.0f && gp.z <= 15.0f;
                    const float ps8[8] = {gp.s, gp.s, gp.s, gp.s, gp.s, gp.s, gp.s, gp.s};
                    const float pr8[8] = {gp.r, gp.r, gp.r, gp.r, gp.r, gp.r, gp.r, gp.r};
                    const float pz8[8] = {gp.z, gp.z, gp.z, gp.z, gp.z, gp.z, gp.z, gp.z};
                    float qv[8];
                    codes8<true>(x, ps8, pr8, pz8, fast, qv);
                    *reinterpret_cast<uint32_t*>(crow + 4 * lane) = pack_codes(qv);
                }
            }
        }

        if (whole) {
            // the K group is one old group: its codes (in the loaded rows) and its scale/zero row
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int r = rg + RPP * i;
                if (r < n) *reinterpret_cast<uint32_t*>(dst.k_codes + (bh * geo.dldq + i0 + r) * (D / 2) + 4 * lane) = raw[i].kc;
            }
            const int64_t si = (bh * geo.ldk + first / G) * D, di = (bh * geo.dldk + j) * D;
            for (int e = tid; e < D / 8; e += kThreads) {
                reinterpret_cast<uint4*>(dst.k_scale + di)[e] = reinterpret_cast<const uint4*>(src.k_scale + si)[e];
                reinterpret_cast<uint4*>(dst.k_zero + di)[e] = reinterpret_cast<const uint4*>(src.k_zero + si)[e];
            }
            return;
        }
        float v[NR][8];
        float mn[8], mx[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) { mn[k] = FLT_MAX; mx[k] = -FLT_MAX; }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            k_values(raw[i], tok[i] < geo.Tq, v[i]);
#pragma unroll
            for (int k = 0; k < 8; ++k) { mn[k] = vmin2(mn[k], v[i][k]); mx[k] = vmax2(mx[k], v[i][k]); }
        }
#pragma unroll
        for (int off = LPR; off < 64; off *= 2) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                mn[k] = vmin2(mn[k], __shfl_xor(mn[k], off));
                mx[k] = vmax2(mx[k], __shfl_xor(mx[k], off));
            }
        }
        if ((tid % 64) < LPR) {
#pragma unroll
            for (int k = 0; k < 8; ++k) { s_mn[wave * D + 8 * lane + k] = mn[k]; s_mx[wave * D + 8 * lane + k] = mx[k]; }
        }
        __syncthreads();
        for (int c = tid; c < D; c += kThreads) {
            float a = s_mn[c], z = s_mx[c];
#pragma unroll
            for (int w = 1; w < NW; ++w) { a = vmin2(a, s_mn[w * D + c]); z = vmax2(z, s_mx[w * D + c]); }
            const GroupParams p = group_params(a, z);
            const int64_t mi = (bh * geo.dldk + j) * D + c;
            dst.k_scale[mi] = p.sb;
            dst.k_zero[mi] = p.zb;
            s_ps[c] = p.s; s_pr[c] = p.r; s_pz[c] = p.z;
        }
        __syncthreads();
        float ps[8], pr[8], pz[8];
        bool fast = true;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            ps[k] = s_ps[8 * lane + k]; pr[k] = s_pr[8 * lane + k]; pz[k] = s_pz[8 * lane + k];
            fast = fast && pz[k] >= 0.0f && pz[k] <= 15.0f;
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = rg + RPP * i;
            if (r < n) {
                float q[8];
                codes8<false>(v[i], ps, pr, pz, fast, q);
                *reinterpret_cast<uint32_t*>(dst.k_codes + (bh * geo.dldq + i0 + r) * (D / 2) + 4 * lane) =
                    pack_codes(q);
            }
        }
        return;
    }
    bid -= nK;
    {
        // ------------------------------ 64 new window rows ------------------------------
        const Bjh ix = split_bjh(bid, H, (uint32_t)geo.nRb);
        const int64_t bh = ix.b * geo.H + ix.h, r0 = ix.j * kTile;
        const int n = (int)min<int64_t>(kTile, geo.R2 - r0);
        const int32_t* kp = keep + bh * geo.K + geo.Tq2 + r0;
        for (int r = rg; r < n; r += RPP) {
            const int64_t t = clamp_tok(kp[r], geo.T);
            const int64_t o = (bh * geo.dldr + r0 + r) * D + 8 * lane;
            if (t >= geo.Tq) {
                const int64_t si = (bh * geo.ldr + (t - geo.Tq)) * D + 8 * lane;
                *reinterpret_cast<uint4*>(dst.k_res + o) = *reinterpret_cast<const uint4*>(src.k_res + si);
                *reinterpret_cast<uint4*>(dst.v_res + o) = *reinterpret_cast<const uint4*>(src.v_res + si);
            } else {
                RowRaw rr;
                load_row<D, G>(src, geo, bh, t, lane, rr);
                float a[8], b[8];
                k_values(rr, true, a);
                v_values(rr, true, b);
                *reinterpret_cast<uint4*>(dst.k_res + o) =
                    make_uint4(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(a[4], a[5]), pack_bf2(a[6], a[7]));
                *reinterpret_cast<uint4*>(dst.v_res + o) =
                    make_uint4(pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3]), pack_bf2(b[4], b[5]), pack_bf2(b[6], b[7]));
            }
        }
    }
}

template <int D, int G>
void launch_evict(const kvq_int4_cache& s, const int32_t* keep, const kvq_int4_cache& d, const EvGeom& geo,
                  int64_t nblk, hipStream_t st) {
    hipLaunchKernelGGL((int4_evict_kernel<D, G>), dim3((unsigned)nblk), dim3(kThreads), 0, st, s, keep, d, geo);
}

// Byte extent of section i of a cache (rows per (b, h) from cap / rcap).
size_t section_bytes(const kvq_int4_cache* c, int i) {
    const int64_t Tq = c->T - c->R, ldq = c->cap ? c->cap : Tq, ldr = c->rcap ? c->rcap : c->R;
    const size_t bh = (size_t)(c->B * c->H), d = (size_t)c->d;
    switch (i) {
    case 0: case 3: return bh * (size_t)ldq * d / 2;
    case 1: case 2: return bh * (size_t)cdiv(ldq, c->g) * d * 2;
    case 4: case 5: return bh * (size_t)ldq * (d / (size_t)c->g) * 2;
    default: return bh * (size_t)ldr * d * 2;
    }
}

const void* section_ptr(const kvq_int4_cache* c, int i) {
    const void* p[8] = {c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero, c->k_res, c->v_res};
    return p[i];
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_int4_evict(const kvq_int4_cache* src, const int32_t* keep, const kvq_int4_cache* dst,
                              kvq_stream stream) {
    int rc = kvq::check_cache_shape(src, "kvq_int4_evict (src)");
    if (rc) return rc;
    rc = kvq::check_cache_shape(dst, "kvq_int4_evict (dst)");
    if (rc) return rc;
    KVQ_REQUIRE(keep, "kvq_int4_evict: NULL keep");
    KVQ_REQUIRE(dst->B == src->B && dst->H == src->H && dst->d == src->d && dst->g == src->g,
                "kvq_int4_evict: dst must have the B, H, d, g of src");
    KVQ_REQUIRE(dst->T <= src->T, "kvq_int4_evict: dst->T (kept tokens, %lld) must be <= src->T (%lld)",
                (long long)dst->T, (long long)src->T);
    // the destination is written while the source is read: no section may overlap
    for (int i = 0; i < 8; ++i) {
        const size_t nd = kvq::section_bytes(dst, i);
        const uintptr_t d0 = reinterpret_cast<uintptr_t>(kvq::section_ptr(dst, i));
        if (!nd || !d0) continue;
        for (int k = 0; k < 8; ++k) {
            const size_t ns = kvq::section_bytes(src, k);
            const uintptr_t s0 = reinterpret_cast<uintptr_t>(kvq::section_ptr(src, k));
            if (!ns || !s0) continue;
            KVQ_REQUIRE(d0 + nd <= s0 || s0 + ns <= d0, "kvq_int4_evict: dst section %d overlaps src section %d", i,
                        k);
        }
    }
    kvq::EvGeom geo;
    geo.T = src->T;
    geo.H = src->H;
    geo.Tq = src->T - src->R;
    geo.ldq = src->cap ? src->cap : geo.Tq;
    geo.ldk = kvq::cdiv(geo.ldq, src->g);
    geo.ldr = src->rcap ? src->rcap : src->R;
    geo.K = dst->T;
    geo.R2 = dst->R;
    geo.Tq2 = dst->T - dst->R;
    geo.dldq = dst->cap ? dst->cap : geo.Tq2;
    geo.dldk = kvq::cdiv(geo.dldq, dst->g);
    geo.dldr = dst->rcap ? dst->rcap : dst->R;
    geo.nKb = kvq::cdiv(geo.Tq2, src->g);
    geo.nRb = kvq::cdiv(geo.R2, kvq::kTile);
    const int64_t nblk = src->B * src->H * (geo.nKb + geo.nRb);
    KVQ_REQUIRE(nblk < ((int64_t)1 << 31), "kvq_int4_evict: grid too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    KVQ_DISPATCH_DG(src->d, src->g, kvq::launch_evict, *src, keep, *dst, geo, nblk, st);
    return kvq::launch_status("kvq_int4_evict");
}
