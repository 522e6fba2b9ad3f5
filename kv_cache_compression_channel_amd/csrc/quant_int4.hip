// quant_int4.hip -- KIVI-style 4-bit affine group quantization of one layer of KV cache,
// its dequantization, and the section sizing.
//
// Explainer (KV cache 压缩：把历史装得更小): quantization section (x ~ s (q - z), bf16 scale
// and bf16 zero per group), grouping-axis section (K grouped per channel across tokens,
// V per token across channels), group-size table (bytes = ceil(N/2) + ceil(N/g)*4) and the
// residual-budget section (the most recent tokens stay bf16).  The integer steps are those
// of the Walkthrough (KV Compression 公式到源码对照) §1.2 with qmin = 0, qmax = 15.
//
// One launch covers K tiles, V tiles and the residual copy.  A tile is one (b, h) and a
// block of consecutive tokens (g tokens for K, or two groups of 32 at g = 32 and d <= 128; 64 for
// V) across all d channels.  The per-row K minima and maxima meet in LDS as bf16 pairs (one dword
// per channel and row slot), which keeps a block within 19 KB and the CU at 7 blocks.  Lane
// layout: d/8 lanes per token row, each owning 8 consecutive channels (one 16-byte load
// of bf16, one 4-byte store of packed codes); a block of NT threads (256, or d*g/32 when that is
// larger, so a K group is at most 4 rows per thread) covers 8*NT/d rows per pass.
// Block order is (b, token block, h) with h fastest, so concurrently running blocks
// read neighbouring token rows of the [B][T][H][d] input.
#include "int4_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kVTile = 64;   // tokens per V tile
constexpr int kResTile = 64; // tokens per residual tile

// Threads per quantizer block: enough that a K group is at most 4 rows per thread (16 bytes
// each), which keeps the tile in registers at no more than about 74 VGPRs.
template <int D, int G>
constexpr int quant_threads() { return D * G / 32 > kThreads ? D * G / 32 : kThreads; }
// Tokens per V tile of the quantizer: 64 per 256 threads, so a larger block also takes a larger
// tile and every thread still quantizes the same number of V elements.
template <int D, int G>
constexpr int quant_vtile() { return kVTile * quant_threads<D, G>() / kThreads; }
// K groups per quantizer block: two at g = 32 (d <= 128), so each thread still carries four rows
// (two at d = 64) and every thread of the block takes a channel of the cross-row reduction.
template <int D, int G>
constexpr int quant_kgroups() { return G == 32 && D <= 128 ? 2 : 1; }

template <int D, int G, int NT = quant_threads<D, G>()>
__global__ void __launch_bounds__(NT) int4_quant_kernel(const uint16_t* __restrict__ K,
                                                              const uint16_t* __restrict__ V, I4Geom geo,
                                                              I4Ptrs out) {
    constexpr int LPR = D / 8;            // lanes per token row
    constexpr int RPP = NT / LPR;         // rows per pass
    constexpr int NGD = D / G;            // V groups per token
    constexpr int VT = quant_vtile<D, G>();   // tokens per V tile
    static_assert(G % RPP == 0 && VT % RPP == 0, "tile shape");
    constexpr int GPB = quant_kgroups<D, G>();   // K groups per block
    constexpr int KT = G * GPB;                  // tokens per K tile
    constexpr int NRG = G / RPP;                 // rows per thread per K group
    constexpr int NR = KT / RPP;                 // rows per thread per K tile
    constexpr int NP = VT * NGD > GPB * D ? VT * NGD : GPB * D;   // parameter slots
    constexpr int NKS = GPB * RPP * D;            // K: one dword per (group, row slot, channel)
    constexpr int NVS = VT * NGD;                 // V: one min and one max per group
    constexpr int NS = NKS > 2 * NVS ? NKS : 2 * NVS;
    // K and V blocks use the one array: a K slot holds the bf16 min (high half) and bf16 max (low
    // half) of its channel, a V block keeps fp32 group minima, then maxima
    __shared__ __attribute__((aligned(16))) uint32_t s_red[NS];
    __shared__ float s_ps[NP], s_pr[NP], s_pz[NP];
    float* const s_mn = reinterpret_cast<float*>(s_red);
    float* const s_mx = s_mn + NVS;

    const int tid = threadIdx.x, lane = tid % LPR, rg = tid / LPR;
    const int64_t H = geo.H, Tq = geo.Tq;
    int64_t bid = blockIdx.x;
    const int64_t nKb = (geo.nKg + GPB - 1) / GPB;   // K tiles per (b, h)
    const int64_t nK = geo.B * nKb * H, nV = geo.B * geo.nVt * H;

    if (bid < nK) {
        // ---------------- K: GPB groups of G tokens, every channel ----------------
        const Bjh ix = split_bjh((uint32_t)bid, (uint32_t)H, (uint32_t)nKb);
        const int64_t h = ix.h, jb = ix.j, b = ix.b;
        const int64_t t0 = jb * KT;
        const int n = (int)min<int64_t>(KT, Tq - t0);
        uint4 raw[NR];
        if (n == KT) {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                raw[i] = ld_stream_u4(K + b * geo.sb + (t0 + rg + RPP * i) * geo.st + h * geo.sh + 8 * lane);
        } else {
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                // rows past the tile's end repeat its last row, which lies in the same group or an
                // earlier one: the last group's min and max are unchanged, and groups wholly past
                // the end are never stored
                const int r = min(rg + RPP * i, n - 1);
                raw[i] = ld_stream_u4(K + b * geo.sb + (t0 + r) * geo.st + h * geo.sh + 8 * lane);
            }
        }
        // per group: min and max over this thread's rows, then every row slot's partials to LDS
        // (two 16-byte stores each), reduced over the RPP slots by the channel threads: no
        // cross-lane permutes
#pragma unroll
        for (int gi = 0; gi < GPB; ++gi) {
            float mn[8], mx[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) { mn[k] = FLT_MAX; mx[k] = -FLT_MAX; }
#pragma unroll
            for (int i = gi * NRG; i < (gi + 1) * NRG; i += 2) {
                float v[8], u[8];
                unpack8(raw[i], v);
                if (i + 1 < (gi + 1) * NRG) unpack8(raw[i + 1], u); else unpack8(raw[i], u);
#pragma unroll
                for (int k = 0; k < 8; ++k) { mn[k] = vmin3(mn[k], v[k], u[k]); mx[k] = vmax3(mx[k], v[k], u[k]); }
            }
            // the input is bf16, so each min and max is a bf16 value (low 16 bits zero): one
            // v_perm_b32 puts both top halves in one dword
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                w[k] = __builtin_amdgcn_perm(__float_as_uint(mn[k]), __float_as_uint(mx[k]), 0x07060302u);
            uint4* pk = reinterpret_cast<uint4*>(s_red + (gi * RPP + rg) * D + 8 * lane);
            pk[0] = make_uint4(w[0], w[1], w[2], w[3]);
            pk[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
        __syncthreads();
        for (int c = tid; c < GPB * D; c += NT) {
            const int gi = c / D, cc = c % D;
            if constexpr (GPB > 1)
                if (gi * G >= n) continue;
            const uint32_t* pk = s_red + gi * RPP * D + cc;
            float a = __uint_as_float(pk[0] & 0xffff0000u), z = __uint_as_float(pk[0] << 16);
#pragma unroll
            for (int w = 1; w < RPP; w += 2) {
                const uint32_t u0 = pk[w * D], u1 = pk[(w + 1 < RPP ? w + 1 : w) * D];
                a = vmin3(a, __uint_as_float(u0 & 0xffff0000u), __uint_as_float(u1 & 0xffff0000u));
                z = vmax3(z, __uint_as_float(u0 << 16), __uint_as_float(u1 << 16));
            }
            const GroupParams p = group_params(a, z);
            const int64_t mi = ((b * H + h) * geo.ldk + jb * GPB + gi) * D + cc;
            out.k_scale[mi] = p.sb;
            out.k_zero[mi] = p.zb;
            s_ps[c] = p.s; s_pr[c] = p.r; s_pz[c] = p.z;
        }
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < GPB; ++gi) {
            float ps[8], pr[8], pz[8];
            bool fast = true;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                ps[k] = s_ps[gi * D + 8 * lane + k]; pr[k] = s_pr[gi * D + 8 * lane + k]; pz[k] = s_pz[gi * D + 8 * lane + k];
                fast = fast && pz[k] >= 0.0f && pz[k] <= 15.0f;
            }
#pragma unroll
            for (int i = gi * NRG; i < (gi + 1) * NRG; ++i) {
                const int r = rg + RPP * i;
                float v[8], q[8];
                unpack8(raw[i], v);
                codes8<false>(v, ps, pr, pz, fast, q);
                if (n == KT || r < n)
                    *reinterpret_cast<uint32_t*>(out.k_codes + ((b * H + h) * geo.ldq + t0 + r) * (D / 2) + 4 * lane) =
                        pack_codes(q);
            }
        }
        return;
    }
    bid -= nK;
    if (bid < nV) {
        // ---------------- V: 64 tokens, groups of G channels per token ----------------
        constexpr int NRV = VT / RPP;
        constexpr int LPG = G / 8;   // lanes per group
        const Bjh ix = split_bjh((uint32_t)bid, (uint32_t)H, (uint32_t)geo.nVt);
        const int64_t h = ix.h, jt = ix.j, b = ix.b;
        const int64_t t0 = jt * VT;
        const int n = (int)min<int64_t>(VT, Tq - t0);
        const int grp = (8 * lane) / G;
        uint4 raw[NRV];
        // every row's load issued before any is used: rows past the tile's end load its last row
        // again (their parameters are never read and their codes never stored)
#pragma unroll
        for (int i = 0; i < NRV; ++i) {
            const int r = rg + RPP * i;
            raw[i] = ld_stream_u4(V + b * geo.sb + (t0 + (r < n ? r : n - 1)) * geo.st + h * geo.sh + 8 * lane);
        }
#pragma unroll
        for (int i = 0; i < NRV; ++i) {
            const int r = rg + RPP * i;
            float mn = FLT_MAX, mx = -FLT_MAX, v[8];
            unpack8(raw[i], v);
            minmax8(v, mn, mx);
            mn = lane_group_reduce<LPG, false>(mn);
            mx = lane_group_reduce<LPG, true>(mx);
            if (lane % LPG == 0) { s_mn[r * NGD + grp] = mn; s_mx[r * NGD + grp] = mx; }
        }
        __syncthreads();
        for (int p = tid; p < n * NGD; p += NT) {
            const GroupParams gp = group_params(s_mn[p], s_mx[p]);
            const int64_t mi = ((b * H + h) * geo.ldq + t0) * NGD + p;
            out.v_scale[mi] = gp.sb;
            out.v_zero[mi] = gp.zb;
            s_ps[p] = gp.s; s_pr[p] = gp.r; s_pz[p] = gp.z;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NRV; ++i) {
            const int r = rg + RPP * i;
            const float ps = s_ps[r * NGD + grp], pr = s_pr[r * NGD + grp], pz = s_pz[r * NGD + grp];
            const bool fast = pz >= 0.0f && pz <= 15.0f;
            const float ps8[8] = {ps, ps, ps, ps, ps, ps, ps, ps}, pr8[8] = {pr, pr, pr, pr, pr, pr, pr, pr};
            const float pz8[8] = {pz, pz, pz, pz, pz, pz, pz, pz};
            float v[8], q[8];
            unpack8(raw[i], v);
            codes8<true>(v, ps8, pr8, pz8, fast, q);
            if (n == VT || r < n)
                *reinterpret_cast<uint32_t*>(out.v_codes + ((b * H + h) * geo.ldq + t0 + r) * (D / 2) + 4 * lane) =
                    pack_codes(q);
        }
        return;
    }
    bid -= nV;
    {
        // ---------------- residual: the last R tokens, verbatim ----------------
        const Bjh ix = split_bjh((uint32_t)bid, (uint32_t)H, (uint32_t)geo.nRt);
        const int64_t h = ix.h, jr = ix.j, b = ix.b;
        const int64_t r0 = jr * kResTile;
        const int n = (int)min<int64_t>(kResTile, geo.R - r0);
        for (int r = rg; r < n; r += RPP) {
            const int64_t src = b * geo.sb + (Tq + r0 + r) * geo.st + h * geo.sh + 8 * lane;
            const int64_t dst = ((b * H + h) * geo.ldr + r0 + r) * D + 8 * lane;
            *reinterpret_cast<uint4*>(out.k_res + dst) = *reinterpret_cast<const uint4*>(K + src);
            *reinterpret_cast<uint4*>(out.v_res + dst) = *reinterpret_cast<const uint4*>(V + src);
        }
    }
}

// Dequantization of one side: x_hat = (q - z) * s rounded once.  q*s and z*s are exact
// in fp32 (4-bit x 8-bit and 8-bit x 8-bit significands), so fma(q, s, -z*s) rounds the
// exact value once.  Residual tokens are copied (bf16) or widened (fp32).
// Tokens per dequantizer tile, K and V alike (a K tile may hold several groups or part of one).
// Short tiles stream the stores best: 32 tokens (two rows per thread at d = 128) measured 1-3%
// faster than 64 at g = 32/64/128 and a third faster than 16 (one row per thread).
constexpr int kDqTile = 32;
// With many heads (d = 128, H a multiple of 4 and at least 32), a tile spans 4 heads and 8
// tokens instead: each wave writes one token's four heads, 1 KB contiguous.  On the full-model
// cache (32 heads) that measured 2-7% faster at g = 32/64/128 (16 tokens: 2-3%); on the decode
// cache (8 heads) the same tiles were 8-11% slower, so fewer heads keep one-head tiles.
constexpr int kDqHeads = 4;
constexpr int kDqTileH = 8;
constexpr int64_t kDqHeadsMinH = 32;
template <int D>
constexpr int dequant_tile() { return kDqTile > kThreads / (D / 8) ? kDqTile : kThreads / (D / 8); }

template <int D, int G, bool IS_K, int OT, int HPT>
__global__ void __launch_bounds__(kThreads) int4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                                const uint16_t* __restrict__ scale,
                                                                const uint16_t* __restrict__ zero,
                                                                const uint16_t* __restrict__ res, I4Geom geo,
                                                                void* __restrict__ out) {
    constexpr int LPR = D / 8;
    constexpr int RPP = kThreads / (LPR * HPT);
    constexpr int TILE = HPT > 1 ? kDqTileH : dequant_tile<D>();   // at least one row per thread
    constexpr int NGT = IS_K && TILE > G ? TILE / G : 1;   // K groups per tile (a tile may hold part of one)
    constexpr int NGD = D / G;
    static_assert(TILE % RPP == 0 && (!IS_K || G % RPP == 0), "tile shape");
    const int tid = threadIdx.x, lane = tid % LPR, rg = tid / (LPR * HPT), hl = (tid / LPR) % HPT;
    const int64_t H = geo.H, T = geo.T, Tq = geo.Tq;
    const int64_t ntile = (Tq + TILE - 1) / TILE;
    int64_t bid = blockIdx.x;
    const int64_t nQ = geo.B * ntile * (H / HPT);

    auto store8 = [&](int64_t t, int64_t b, int64_t h, const float (&v)[8]) {
        const int64_t o = ((b * T + t) * H + h) * D + 8 * lane;
        if constexpr (OT == KVQ_FP32) {
            float* p = static_cast<float*>(out) + o;
            st_stream_f4(p, make_float4(v[0], v[1], v[2], v[3]));
            st_stream_f4(p + 4, make_float4(v[4], v[5], v[6], v[7]));
        } else {
            uint16_t* p = static_cast<uint16_t*>(out) + o;
            st_stream_u4(p, make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                       pack_bf2(v[6], v[7])));
        }
    };

    if (bid < nQ) {
        const Bjh ix = split_bjh((uint32_t)bid, (uint32_t)(H / HPT), (uint32_t)ntile);
        const int64_t h = ix.h * HPT + hl, j = ix.j, b = ix.b;
        const int64_t t0 = j * TILE;
        const int n = (int)min<int64_t>(TILE, Tq - t0);
        float s8[NGT][8], zs8[NGT][8];
        if constexpr (IS_K) {
#pragma unroll
            for (int q = 0; q < NGT; ++q) {
                // a group past the last is never used (its rows are past n); its index is clamped
                const int64_t jq = min<int64_t>((j * TILE) / G + q, geo.nKg - 1);
                const int64_t mi = ((b * H + h) * geo.ldk + jq) * D + 8 * lane;
                const uint4 sv = *reinterpret_cast<const uint4*>(scale + mi);
                const uint4 zv = *reinterpret_cast<const uint4*>(zero + mi);
                float zf[8];
                unpack8(sv, s8[q]);
                unpack8(zv, zf);
#pragma unroll
                for (int k = 0; k < 8; ++k) zs8[q][k] = -zf[k] * s8[q][k];
            }
        }
        // Every row's words are loaded before any is used (one round trip per block).  A row past n
        // (the last tile's tail) takes row n - 1 for its loads and its store alike and writes that
        // row's values again (a K row past n has the parameters of row n - 1's group: a group of
        // the tile past the last one repeats the last), so no load or store sits behind a branch.
        constexpr int NRW = TILE / RPP;
        uint32_t wr[NRW];
        uint16_t sr[NRW], zr[NRW];
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
            const int64_t t = t0 + min(rg + RPP * i, n - 1);
            wr[i] = __builtin_nontemporal_load(
                reinterpret_cast<const uint32_t*>(codes + ((b * H + h) * geo.ldq + t) * (D / 2) + 4 * lane));
            if constexpr (!IS_K) {
                const int64_t mi = ((b * H + h) * geo.ldq + t) * NGD + (8 * lane) / G;
                sr[i] = scale[mi];
                zr[i] = zero[mi];
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // every load issued before the first store
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
            const int r = rg + RPP * i;
            const int q = IS_K ? (RPP * i) / G : 0;   // the row's group inside the tile (RPP divides G)
            const int64_t t = t0 + min(r, n - 1);
            const uint32_t w = wr[i];
            // nibbles 2e and 2e+1 sit in byte e of w & 0x0f0f0f0f and of (w >> 4) & 0x0f0f0f0f;
            // each byte converts with one v_cvt_f32_ubyte<e>
            const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
            float c[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[2 * e] = (float)((lo >> (8 * e)) & 0xffu);
                c[2 * e + 1] = (float)((hi >> (8 * e)) & 0xffu);
            }
            float v[8];
            if constexpr (IS_K) {
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(c[k], s8[q][k], zs8[q][k]);
            } else {
                const float s = bf_to_f(sr[i]);
                const float zs = -bf_to_f(zr[i]) * s;
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(c[k], s, zs);
            }
            store8(t, b, h, v);
        }
        return;
    }
    bid -= nQ;
    const Bjh ix = split_bjh((uint32_t)bid, (uint32_t)H, (uint32_t)geo.nRt);
    const int64_t h = ix.h, jr = ix.j, b = ix.b;
    const int64_t r0 = jr * kResTile;
    const int n = (int)min<int64_t>(kResTile, geo.R - r0);
    constexpr int RPP1 = kThreads / LPR;
    for (int r = tid / LPR; r < n; r += RPP1) {
        const uint4 a = *reinterpret_cast<const uint4*>(res + ((b * H + h) * geo.ldr + r0 + r) * D + 8 * lane);
        if constexpr (OT == KVQ_BF16) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + ((b * T + Tq + r0 + r) * H + h) * D + 8 * lane) = a;
        } else {
            float v[8];
            unpack8(a, v);
            store8(Tq + r0 + r, b, h, v);
        }
    }
}

// Streaming append, residual side.  mode 0: rows R .. R+n-1 of each (b, h) residual receive the
// n new tokens (new is [B][n][H][d]).  mode 1: rows g .. m-1 move down to 0 .. m-g-1, in
// ascending chunks of at most g rows, each read completely (barrier) before it is written, so
// no row is overwritten before it has been read.  One workgroup per (b, h); K and V together.
template <int D>
__global__ void __launch_bounds__(kThreads) int4_residual_kernel(uint16_t* __restrict__ k_res,
                                                                 uint16_t* __restrict__ v_res,
                                                                 const uint16_t* __restrict__ k_new,
                                                                 const uint16_t* __restrict__ v_new, int64_t H,
                                                                 int64_t ldr, int64_t R, int64_t n, int64_t g,
                                                                 int64_t m, int mode) {
    constexpr int LPR = D / 8;
    constexpr int RPP = kThreads / LPR;
    const int tid = threadIdx.x, lane = tid % LPR, rg = tid / LPR;
    const int64_t bh = blockIdx.x, b = bh / H, h = bh % H;
    uint16_t* kr = k_res + bh * ldr * D + 8 * lane;
    uint16_t* vr = v_res + bh * ldr * D + 8 * lane;
    if (mode == 0) {
        for (int64_t i = rg; i < n; i += RPP) {
            const int64_t src = ((b * n + i) * H + h) * D + 8 * lane;
            *reinterpret_cast<uint4*>(kr + (R + i) * D) = *reinterpret_cast<const uint4*>(k_new + src);
            *reinterpret_cast<uint4*>(vr + (R + i) * D) = *reinterpret_cast<const uint4*>(v_new + src);
        }
        return;
    }
    // chunk of RPP rows (RPP <= 32 <= g): read rows c0 + g + rg, barrier, write rows c0 + rg
    for (int64_t c0 = 0; c0 < m - g; c0 += RPP) {
        const int64_t i = c0 + rg;
        uint4 ka = {0u, 0u, 0u, 0u}, va = {0u, 0u, 0u, 0u};
        if (i < m - g) {
            ka = *reinterpret_cast<const uint4*>(kr + (i + g) * D);
            va = *reinterpret_cast<const uint4*>(vr + (i + g) * D);
        }
        __syncthreads();
        if (i < m - g) {
            *reinterpret_cast<uint4*>(kr + i * D) = ka;
            *reinterpret_cast<uint4*>(vr + i * D) = va;
        }
        __syncthreads();
    }
}

I4Geom geom_of(const kvq_int4_cache* c) {
    I4Geom g;
    g.B = c->B; g.T = c->T; g.H = c->H; g.d = c->d; g.g = c->g; g.R = c->R;
    g.Tq = c->T - c->R;
    g.nKg = cdiv(g.Tq, g.g);
    g.nVt = cdiv(g.Tq, kVTile);
    g.ldq = c->cap ? c->cap : g.Tq;
    g.ldk = cdiv(g.ldq, g.g);
    g.ldr = c->rcap ? c->rcap : g.R;
    g.st = g.H * g.d;
    g.sh = g.d;
    g.sb = g.T * g.st;
    g.nRt = cdiv(g.R, kResTile);
    return g;
}

// nblk is the grid at one K group and 64 tokens per tile (what the callers check); the quantizer's
// own K and V tiles may be larger, which only shrinks its grid.
template <int D, int G>
void launch_quant(const uint16_t* K, const uint16_t* V, const I4Geom& g, const I4Ptrs& p, int64_t nblk,
                  hipStream_t st) {
    (void)nblk;
    I4Geom gq = g;
    gq.nVt = cdiv(g.Tq, (int64_t)quant_vtile<D, G>());
    const int64_t n = gq.B * gq.H * (cdiv(gq.nKg, (int64_t)quant_kgroups<D, G>()) + gq.nVt + gq.nRt);
    hipLaunchKernelGGL((int4_quant_kernel<D, G>), dim3((unsigned)n), dim3(quant_threads<D, G>()), 0, st, K, V, gq, p);
}

template <int D, int G, int HPT>
void launch_dequant_h(bool is_k, int ot, const kvq_int4_cache* c, const I4Geom& g, void* out, hipStream_t st) {
    constexpr int TILE = HPT > 1 ? kDqTileH : dequant_tile<D>();
    const int64_t nblk = g.B * (cdiv(g.Tq, (int64_t)TILE) * (g.H / HPT) + g.H * g.nRt);
    const dim3 grid((unsigned)nblk), blk(kThreads);
    if (is_k) {
        if (ot == KVQ_FP32)
            hipLaunchKernelGGL((int4_dequant_kernel<D, G, true, KVQ_FP32, HPT>), grid, blk, 0, st, c->k_codes, c->k_scale,
                               c->k_zero, c->k_res, g, out);
        else
            hipLaunchKernelGGL((int4_dequant_kernel<D, G, true, KVQ_BF16, HPT>), grid, blk, 0, st, c->k_codes, c->k_scale,
                               c->k_zero, c->k_res, g, out);
    } else {
        if (ot == KVQ_FP32)
            hipLaunchKernelGGL((int4_dequant_kernel<D, G, false, KVQ_FP32, HPT>), grid, blk, 0, st, c->v_codes, c->v_scale,
                               c->v_zero, c->v_res, g, out);
        else
            hipLaunchKernelGGL((int4_dequant_kernel<D, G, false, KVQ_BF16, HPT>), grid, blk, 0, st, c->v_codes, c->v_scale,
                               c->v_zero, c->v_res, g, out);
    }
}
template <int D, int G>
void launch_dequant(bool is_k, int ot, const kvq_int4_cache* c, const I4Geom& g, void* out, hipStream_t st) {
    if (D == 128 && g.H % kDqHeads == 0 && g.H >= kDqHeadsMinH) launch_dequant_h<D, G, kDqHeads>(is_k, ot, c, g, out, st);
    else launch_dequant_h<D, G, 1>(is_k, ot, c, g, out, st);
}


}  // namespace

int check_cache_shape(const kvq_int4_cache* c, const char* name) {
    KVQ_REQUIRE(c, "%s: NULL cache descriptor", name);
    KVQ_REQUIRE(c->B >= 1 && c->T >= 1 && c->H >= 1, "%s: B, T, H must be >= 1", name);
    KVQ_REQUIRE(c->d == 64 || c->d == 128 || c->d == 256, "%s: d must be 64, 128 or 256 (got %lld)", name,
                (long long)c->d);
    KVQ_REQUIRE((c->g == 32 || c->g == 64 || c->g == 128) && c->g <= c->d,
                "%s: g must be 32, 64 or 128 and <= d (got %lld)", name, (long long)c->g);
    KVQ_REQUIRE(c->R >= 0 && c->R <= c->T, "%s: need 0 <= R <= T", name);
    KVQ_REQUIRE(c->B * c->T * c->H * c->d < ((int64_t)1 << 40), "%s: cache too large", name);
    const int64_t Tq = c->T - c->R;
    KVQ_REQUIRE(c->cap == 0 || (c->cap >= Tq && c->cap % c->g == 0),
                "%s: cap (%lld) must be 0 or a multiple of g that is >= T - R (%lld)", name, (long long)c->cap,
                (long long)Tq);
    KVQ_REQUIRE(c->rcap == 0 || c->rcap >= c->R, "%s: rcap (%lld) must be 0 or >= R (%lld)", name,
                (long long)c->rcap, (long long)c->R);
    const void* ptrs[8] = {c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero, c->k_res, c->v_res};
    const char* names[8] = {"k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_res", "v_res"};
    for (int i = 0; i < 8; ++i) {
        const bool needed = (i < 6) ? Tq > 0 : c->R > 0;
        KVQ_REQUIRE(!needed || ptrs[i], "%s: NULL %s", name, names[i]);
        KVQ_REQUIRE_ALIGNED(ptrs[i], names[i]);
    }
    return KVQ_OK;
}

int dequant_int4(const kvq_int4_cache* c, bool is_k, void* out, int ot, hipStream_t st) {
    const int rc = check_cache_shape(c, "kvq_dequant");
    if (rc) return rc;
    KVQ_REQUIRE(out, "kvq_dequant: NULL out");
    KVQ_REQUIRE(ot == KVQ_FP32 || ot == KVQ_BF16, "kvq_dequant: ot must be KVQ_FP32 or KVQ_BF16");
    KVQ_REQUIRE_ALIGNED(out, "out");
    const I4Geom g = geom_of(c);
    KVQ_REQUIRE(g.B * g.H * ((is_k ? g.nKg : g.nVt) + g.nRt) < ((int64_t)1 << 31), "kvq_dequant: grid too large");
    KVQ_DISPATCH_DG(c->d, c->g, launch_dequant, is_k, ot, c, g, out, st);
    return launch_status("INT4 dequantization");
}

}  // namespace kvq

extern "C" {

int kvq_int4_cache_sizes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, int64_t R, size_t sect_bytes[8],
                         size_t* total) {
    KVQ_REQUIRE(sect_bytes && total, "kvq_int4_cache_sizes: NULL output");
    KVQ_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 2 && d % 2 == 0 && g >= 1 && d % g == 0 && R >= 0 && R <= T,
                "kvq_int4_cache_sizes: invalid shape");
    const size_t bh = (size_t)(B * H), Tq = (size_t)(T - R);
    sect_bytes[0] = bh * Tq * (size_t)(d / 2);
    sect_bytes[1] = bh * (size_t)kvq::cdiv((int64_t)Tq, g) * (size_t)d * 2;
    sect_bytes[2] = sect_bytes[1];
    sect_bytes[3] = sect_bytes[0];
    sect_bytes[4] = bh * Tq * (size_t)(d / g) * 2;
    sect_bytes[5] = sect_bytes[4];
    sect_bytes[6] = bh * (size_t)R * (size_t)d * 2;
    sect_bytes[7] = sect_bytes[6];
    size_t t = 0;
    for (int i = 0; i < 8; ++i) t += sect_bytes[i];
    *total = t;
    return KVQ_OK;
}

int kvq_group_quant_int4(const void* K, const void* V, const kvq_int4_cache* c, kvq_stream stream) {
    const int rc = kvq::check_cache_shape(c, "kvq_group_quant_int4");
    if (rc) return rc;
    KVQ_REQUIRE(K && V, "kvq_group_quant_int4: NULL K or V");
    KVQ_REQUIRE_ALIGNED(K, "K");
    KVQ_REQUIRE_ALIGNED(V, "V");
    const kvq::I4Geom g = kvq::geom_of(c);
    const kvq::I4Ptrs p{c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero, c->k_res, c->v_res};
    const int64_t nblk = g.B * g.H * (g.nKg + g.nVt + g.nRt);
    KVQ_REQUIRE(nblk < ((int64_t)1 << 31), "kvq_group_quant_int4: grid too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    KVQ_DISPATCH_DG(c->d, c->g, kvq::launch_quant, static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                    g, p, nblk, st);
    return kvq::launch_status("INT4 group quantization");
}

int kvq_int4_append(kvq_int4_cache* c, const void* k_new, const void* v_new, int64_t n, int64_t r_keep,
                    kvq_stream stream) {
    KVQ_REQUIRE(c, "kvq_int4_append: NULL cache descriptor");
    KVQ_REQUIRE(k_new && v_new, "kvq_int4_append: NULL k_new or v_new");
    KVQ_REQUIRE(c->B >= 1 && c->H >= 1 && c->T >= 0 && c->R >= 0 && c->R <= c->T,
                "kvq_int4_append: need B, H >= 1 and 0 <= R <= T");
    KVQ_REQUIRE(c->d == 64 || c->d == 128 || c->d == 256, "kvq_int4_append: d must be 64, 128 or 256");
    KVQ_REQUIRE((c->g == 32 || c->g == 64 || c->g == 128) && c->g <= c->d,
                "kvq_int4_append: g must be 32, 64 or 128 and <= d");
    KVQ_REQUIRE(c->cap > 0 && c->rcap > 0, "kvq_int4_append: the cache needs cap and rcap (a growable layout)");
    const int64_t g = c->g, Tq = c->T - c->R;
    KVQ_REQUIRE(Tq % g == 0 && c->cap % g == 0 && Tq <= c->cap,
                "kvq_int4_append: T - R (%lld) and cap (%lld) must be multiples of g with T - R <= cap",
                (long long)Tq, (long long)c->cap);
    KVQ_REQUIRE(n >= 1 && n <= g, "kvq_int4_append: 1 <= n <= g (got n = %lld)", (long long)n);
    KVQ_REQUIRE(r_keep >= 0 && c->R < r_keep + g,
                "kvq_int4_append: need r_keep >= 0 and R (%lld) < r_keep + g", (long long)c->R);
    const bool flush = c->R + n >= r_keep + g;
    KVQ_REQUIRE(c->R + n <= c->rcap, "kvq_int4_append: rcap (%lld) < R + n (%lld)", (long long)c->rcap,
                (long long)(c->R + n));
    KVQ_REQUIRE(!flush || Tq + g <= c->cap, "kvq_int4_append: cap (%lld) full", (long long)c->cap);
    KVQ_REQUIRE(c->B * c->T * c->H * c->d < ((int64_t)1 << 40), "kvq_int4_append: cache too large");
    const void* ptrs[8] = {c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero, c->k_res, c->v_res};
    for (int i = 0; i < 8; ++i) {
        KVQ_REQUIRE(ptrs[i], "kvq_int4_append: NULL section pointer");
        KVQ_REQUIRE_ALIGNED(ptrs[i], "section");
    }
    KVQ_REQUIRE_ALIGNED(k_new, "k_new");
    KVQ_REQUIRE_ALIGNED(v_new, "v_new");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t H = c->H, R = c->R, m = R + n;
    const dim3 rgrid((unsigned)(c->B * H)), blk(kvq::kThreads);
    const uint16_t* kn = static_cast<const uint16_t*>(k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(v_new);
#define KVQ_RES_LAUNCH(DD, MODE)                                                                              \
    hipLaunchKernelGGL((kvq::int4_residual_kernel<DD>), rgrid, blk, 0, st, c->k_res, c->v_res, kn, vn, H, c->rcap, \
                       R, n, g, m, MODE)
    // 1) the new tokens go after the residual
    if (c->d == 64) KVQ_RES_LAUNCH(64, 0);
    else if (c->d == 128) KVQ_RES_LAUNCH(128, 0);
    else KVQ_RES_LAUNCH(256, 0);
    if (flush) {
        // 2) the oldest g residual rows become K group Tq / g and V rows Tq .. Tq + g - 1: the batch
        //    quantizer over a g-token input read from the residual section ([B][H][rcap][d])
        kvq_int4_cache f = *c;
        f.T = g;
        f.R = 0;
        f.k_codes = c->k_codes + Tq * (c->d / 2);
        f.v_codes = c->v_codes + Tq * (c->d / 2);
        f.k_scale = c->k_scale + (Tq / g) * c->d;
        f.k_zero = c->k_zero + (Tq / g) * c->d;
        f.v_scale = c->v_scale + Tq * (c->d / g);
        f.v_zero = c->v_zero + Tq * (c->d / g);
        kvq::I4Geom geo = kvq::geom_of(&f);
        geo.ldq = c->cap;
        geo.ldk = c->cap / g;
        geo.ldr = c->rcap;
        geo.sb = H * c->rcap * c->d;
        geo.st = c->d;
        geo.sh = c->rcap * c->d;
        const kvq::I4Ptrs p{f.k_codes, f.k_scale, f.k_zero, f.v_codes, f.v_scale, f.v_zero, f.k_res, f.v_res};
        const int64_t nblk = geo.B * geo.H * (geo.nKg + geo.nVt + geo.nRt);
        KVQ_DISPATCH_DG(c->d, g, kvq::launch_quant, c->k_res, c->v_res, geo, p, nblk, st);
        // 3) the rest of the residual moves down by g rows
        if (c->d == 64) KVQ_RES_LAUNCH(64, 1);
        else if (c->d == 128) KVQ_RES_LAUNCH(128, 1);
        else KVQ_RES_LAUNCH(256, 1);
    }
#undef KVQ_RES_LAUNCH
    const int rc = kvq::launch_status("kvq_int4_append");
    if (rc) return rc;
    c->T += n;
    c->R = flush ? m - g : m;
    return KVQ_OK;
}

}  // extern "C"
