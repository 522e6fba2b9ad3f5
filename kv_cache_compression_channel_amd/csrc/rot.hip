// rot.hip -- the Hadamard-rotated per-token 4-bit cache: quantization, dequantization and GQA
// decode attention.
//
// KV-COBRA notes (papernotes.org), item 4 on the Walsh-Hadamard rotation: an orthogonal
// Walsh-Hadamard matrix with a fixed random sign flip mixes the coordinates of every vector,
// so each coordinate carries the mean variance and outlier channels disappear before scalar
// quantization; the comparison with QuaRot / TurboQuant names the same rotation idea.  The
// calibration-free form built here: y = (1/sqrt(d)) H_d (s (.) x), H_d the Sylvester Hadamard
// matrix, s the caller's signs (one vector for K, one for V), then per-token 4-bit groups of g
// rotated coordinates with the group steps of the KIVI quantizer (Explainer, quantization
// section).  Attention runs in the rotated space: q' = R_K q, o' = softmax(q' . k') v', and
// the output is R_V^-1 o' (orthogonality keeps q . k = q' . k').
//
// The transform is butterflies in a fixed order, stage h = 1, 2, 4, ..., d/2, each pair
// (j, j + h) becoming (a + b, a - b) in fp32, then one multiply by fp32(1/sqrt(d)).  Lane
// layout for token rows: d/8 lanes per row, 8 consecutive coordinates per lane, so stages 1, 2, 4
// run inside a lane and stages 8 .. d/2 across lanes (xor shuffles inside the row's lanes).
#include <cmath>

#include "int4_common.h"

namespace kvq {
void launch_attn_mfma_rot(const kvq_rot_cache* c, const float* qrot, int64_t Hq, float* ws, int nsplit,
                          int64_t split_len, hipStream_t st);

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;
constexpr int kWaves = kThreads / 64;
constexpr float kNegBig = -3.0e38f;

struct SignBits {
    uint32_t w[8];   // bit c of the d-bit mask: coordinate c is negated
};

// Bits c0 .. c0+7 (c0 % 8 == 0).  The word is picked by a select over the eight values: an index
// that differs between lanes would read the argument from kernel-argument memory, once per lane,
// in front of the first use.
__device__ __forceinline__ uint32_t sign8(const SignBits& s, int c0) {
    const int wi = c0 / 32;
    uint32_t w = __builtin_amdgcn_readfirstlane(s.w[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) w = wi == i ? __builtin_amdgcn_readfirstlane(s.w[i]) : w;
    return (w >> (c0 % 32)) & 0xffu;
}

// x from the lane whose index differs in bit pattern M (M < 32): ds_swizzle's bit mode, which
// needs no address computation.
template <int M>
__device__ __forceinline__ float swz_xor(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1f | (M << 10)));
}

template <int M, int LPR>
__device__ __forceinline__ void fwht_cross(float (&v)[8], int lane) {
    if constexpr (M < LPR) {
        // low lane of the pair: own + partner; high lane: partner - own.  fma(+-1, own, partner)
        // rounds exactly like that addition or subtraction.
        const float sg = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(sg, v[k], swz_xor<M>(v[k]));
        fwht_cross<2 * M, LPR>(v, lane);
    }
}

// Butterflies of one row held as 8 consecutive coordinates per lane, LPR lanes per row.
template <int LPR>
__device__ __forceinline__ void fwht_row(float (&v)[8], int lane) {
#pragma unroll
    for (int h = 1; h < 8; h *= 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j & h) continue;
            const float a = v[j], b = v[j + h];
            v[j] = a + b;
            v[j + h] = a - b;
        }
    }
    fwht_cross<1, LPR>(v, lane);
}

struct RotGeom {
    int64_t B, T, H;
    float c;        // fp32(1 / sqrt(d))
    uint32_t rows;  // B * T * H
    uint32_t ntt;   // token tiles of kRowsPerBlock per (b, h)
};

// Block u of the quantizer and dequantizer grids: (b, token tile, h) with h fastest, so blocks
// running together touch neighbouring [B][T][H] input rows; the index arithmetic is done once
// per block instead of per row.
struct RotTile {
    int64_t in0;    // [B][T][H] row of the tile's first token
    int64_t out0;   // [B][H][T] row of the tile's first token
    int n;          // tokens in the tile
};
__device__ __forceinline__ RotTile rot_tile(const RotGeom& geo, uint32_t u) {
    const uint32_t H = (uint32_t)geo.H;
    const uint32_t q = u / H, h = u - q * H;
    const uint32_t b = q / geo.ntt, tt = q - b * geo.ntt;
    const int64_t t0 = (int64_t)tt * kRowsPerBlock;
    RotTile r;
    r.in0 = ((int64_t)b * geo.T + t0) * geo.H + h;
    r.out0 = ((int64_t)b * geo.H + h) * geo.T + t0;
    r.n = (int)min<int64_t>(kRowsPerBlock, geo.T - t0);
    return r;
}

// ---------------- quantization: K and V rows of the [B][T][H][d] input ----------------
// Each thread loads the K and V pieces of all its rows first (rows past the end repeat the last
// row and are not stored, so every lane takes part in every shuffle), then rotates them.  The
// sign flips are applied to the bf16 pairs before widening (one xor per pair of coordinates).
// Group parameters are computed once per group rather than in each of its lanes: the group's
// first lane puts the group's (min, max) in its wave's LDS table, lane j of the wave computes
// the parameters of table entries j, j + 64, ... (and stores the bf16 scale and zero), and every
// lane reads back the entries of its own groups.  The table is private to the wave, so no block
// barrier is needed.  Rows are taken in batches of SB sides (K and V together when d <= 128),
// which bounds the rotated values held in registers to SB * NR rows of 8.
template <int D, int G>
__global__ void __launch_bounds__(kThreads) rot_quant_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                            RotGeom geo, SignBits ks, SignBits vs, kvq_rot_cache out) {
    constexpr int LPR = D / 8, RPP = kThreads / LPR, LPG = G / 8, NGD = D / G, NR = kRowsPerBlock / RPP;
    constexpr int RW = 64 / LPR;              // rows of a wave in one pass
    constexpr int GW = RW * NGD;              // groups of a wave in one row of each of its lanes
    constexpr int SB = D <= 128 ? 2 : 1;      // sides per batch
    constexpr int NRS = SB * NR;              // rows per lane in a batch
    constexpr int NPAIR = NRS * GW;           // groups of a wave in a batch
    __shared__ float2 s_mm[kWaves][NPAIR];
    __shared__ float4 s_prm[kWaves][NPAIR];
    const int tid = threadIdx.x, lane = tid % LPR, rg = tid / LPR;
    const int wl = tid % 64, wv = tid / 64;
    const int gw = wl / LPG;                  // this lane's group in the wave's table row
    const RotTile tl = rot_tile(geo, blockIdx.x);
    const int64_t rs_in = geo.H * D;          // elements between consecutive tokens of the input
    uint4 raw[2][NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int u = min(rg + RPP * i, tl.n - 1);
        const int64_t e = (tl.in0 * D + 8 * lane) + u * rs_in;
        raw[0][i] = *reinterpret_cast<const uint4*>(K + e);
        raw[1][i] = *reinterpret_cast<const uint4*>(V + e);
    }
    // bf16 pair j of the lane holds coordinates 8 lane + 2j (bits 0..15) and + 2j + 1 (bits 16..31)
    uint32_t sm[2][4];
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        const uint32_t s8 = sign8(side ? vs : ks, 8 * lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm[side][j] = ((s8 >> (2 * j)) & 1u) << 15 | ((s8 >> (2 * j + 1)) & 1u) << 31;
    }
#pragma unroll
    for (int s0 = 0; s0 < 2; s0 += SB) {
        float v[NRS][8];
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
            const int side = s0 + rs / NR, i = rs % NR;
            uint4 w = raw[side][i];
            w.x ^= sm[side][0]; w.y ^= sm[side][1]; w.z ^= sm[side][2]; w.w ^= sm[side][3];
            unpack8(w, v[rs]);
            fwht_row<LPR>(v[rs], lane);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[rs][k] = v[rs][k] * geo.c;
            float mn = vmin3(v[rs][0], v[rs][1], v[rs][2]), mx = vmax3(v[rs][0], v[rs][1], v[rs][2]);
            mn = vmin3(mn, v[rs][3], v[rs][4]); mx = vmax3(mx, v[rs][3], v[rs][4]);
            mn = vmin3(mn, v[rs][5], v[rs][6]); mx = vmax3(mx, v[rs][5], v[rs][6]);
            mn = vmin2(mn, v[rs][7]); mx = vmax2(mx, v[rs][7]);
            mn = lane_group_reduce<LPG, false>(mn);
            mx = lane_group_reduce<LPG, true>(mx);
            if (wl % LPG == 0) s_mm[wv][rs * GW + gw] = make_float2(mn, mx);
        }
        __builtin_amdgcn_wave_barrier();
        // one group per lane: parameters, and the bf16 scale / zero of the group
#pragma unroll
        for (int p0 = 0; p0 < NPAIR; p0 += 64) {
            const int p = p0 + wl;
            if (NPAIR % 64 == 0 || p < NPAIR) {
                const float2 m = s_mm[wv][p];
                const GroupParams gp = group_params(m.x, m.y);
                s_prm[wv][p] = make_float4(gp.s, gp.r, gp.z, 0.0f);
                const int rs = p / GW, gq = p % GW;
                const int side = s0 + rs / NR, i = rs % NR;
                const int u = wv * RW + gq / NGD + RPP * i;
                if (u < tl.n) {
                    const int64_t mi = (tl.out0 + u) * NGD + gq % NGD;
                    (side ? out.v_scale : out.k_scale)[mi] = gp.sb;
                    (side ? out.v_zero : out.k_zero)[mi] = gp.zb;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
            const int side = s0 + rs / NR, i = rs % NR;
            const float4 pp = s_prm[wv][rs * GW + gw];
            const bool fast = pp.z >= 0.0f && pp.z <= 15.0f;
            const float ps8[8] = {pp.x, pp.x, pp.x, pp.x, pp.x, pp.x, pp.x, pp.x};
            const float pr8[8] = {pp.y, pp.y, pp.y, pp.y, pp.y, pp.y, pp.y, pp.y};
            const float pz8[8] = {pp.z, pp.z, pp.z, pp.z, pp.z, pp.z, pp.z, pp.z};
            float q[8];
            codes8<true>(v[rs], ps8, pr8, pz8, fast, q);
            const int u = rg + RPP * i;
            if (u < tl.n)
                *reinterpret_cast<uint32_t*>((side ? out.v_codes : out.k_codes) + (tl.out0 + u) * (D / 2) + 4 * lane) =
                    pack_codes(q);
        }
        __builtin_amdgcn_wave_barrier();   // the table is reused by the next batch
    }
}

// ---------------- dequantization of one side back to the original coordinates ----------------
// Loads of all the thread's rows first (rows past the end repeat the last row, not stored).
template <int D, int G, int OT>
__global__ void __launch_bounds__(kThreads) rot_dequant_kernel(const uint8_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ scale,
                                                              const uint16_t* __restrict__ zero, RotGeom geo,
                                                              SignBits sg, void* __restrict__ out) {
    constexpr int LPR = D / 8, RPP = kThreads / LPR, NGD = D / G, NR = kRowsPerBlock / RPP;
    const int tid = threadIdx.x, lane = tid % LPR, rg = tid / LPR;
    const RotTile tl = rot_tile(geo, blockIdx.x);
    const uint32_t sb = sign8(sg, 8 * lane);
    uint32_t w[NR];
    uint16_t sc[NR], zr[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t o = tl.out0 + min(rg + RPP * i, tl.n - 1);   // [B][H][T] cache row
        w[i] = *reinterpret_cast<const uint32_t*>(codes + o * (D / 2) + 4 * lane);
        const int64_t mi = o * NGD + (8 * lane) / G;
        sc[i] = scale[mi];
        zr[i] = zero[mi];
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int u = rg + RPP * i;
        const float s = bf_to_f(sc[i]), zs = -bf_to_f(zr[i]) * s;
        const uint32_t lo = w[i] & 0x0f0f0f0fu, hi = (w[i] >> 4) & 0x0f0f0f0fu;
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __builtin_fmaf((float)((lo >> (8 * e)) & 0xffu), s, zs);
            v[2 * e + 1] = __builtin_fmaf((float)((hi >> (8 * e)) & 0xffu), s, zs);
        }
        fwht_row<LPR>(v, lane);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float x = v[k] * geo.c;
            v[k] = ((sb >> k) & 1u) ? -x : x;
        }
        if (u >= tl.n) continue;
        const int64_t r = tl.in0 + u * geo.H;                          // [B][T][H] output row
        if constexpr (OT == KVQ_FP32) {
            float* p = static_cast<float*>(out) + r * D + 8 * lane;
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + r * D + 8 * lane) =
                make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
        }
    }
}

// ---------------- decode attention ----------------
struct RotAttnArgs {
    const uint8_t* k_codes;
    const uint16_t* k_scale;
    const uint16_t* k_zero;
    const uint8_t* v_codes;
    const uint16_t* v_scale;
    const uint16_t* v_zero;
    const uint16_t* q;
    float* qr;        // rotated queries [B][Hq][D] fp32, times sm_scale * log2(e)
    float* part;      // split partials [B*Hq][nsplit][D + 2]
    void* out;
    int64_t B, T, H, Hq;
    int64_t split_len;
    int nsplit;
    int nqg;          // blocks per (b, h, split): query heads of a KV head in groups of at most 8
    float c;
    float qscale;
};

// q' = R_K q (fp32 butterflies) times sm_scale * log2(e); one row per D/8 lanes.
template <int D>
__global__ void __launch_bounds__(kThreads) rot_q_kernel(RotAttnArgs a, SignBits ks) {
    constexpr int LPR = D / 8, RPP = kThreads / LPR;
    const int tid = threadIdx.x, lane = tid % LPR;
    const int64_t r = (int64_t)blockIdx.x * RPP + tid / LPR;
    if (r >= a.B * a.Hq) return;   // a whole row's lanes leave together
    const uint32_t sb = sign8(ks, 8 * lane);
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(a.q + r * D + 8 * lane), v);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ((sb >> k) & 1u) ? -v[k] : v[k];
    fwht_row<LPR>(v, lane);
    float* p = a.qr + r * D + 8 * lane;
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = v[k] * a.c * a.qscale;
}

// One block per (b, h, query group, token split): NQ (at most 8) of the query heads of KV head h
// (16 heads per KV head take two groups, so each thread keeps 8 heads' accumulators).  Per token, each lane
// dequantizes its 8 rotated K coordinates (one group scale and zero) and its 8 V coordinates;
// dot products finish with butterfly shuffles over the token's lanes; online softmax in the
// base-2 domain; the split writes (max, sum, acc[D]) per query head.
template <int D, int GS, int NQ>
__global__ void __launch_bounds__(kThreads) rot_attn_split_kernel(const RotAttnArgs a) {
    constexpr int LPT = D / 8, TPW = 64 / LPT, TPS = TPW * kWaves, NGD = D / GS;
    __shared__ float s_m[kWaves][NQ], s_l[kWaves][NQ];
    __shared__ float s_acc[kWaves][NQ][D];
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int li = lane % LPT, tg = lane / LPT;
    const int64_t bhg = blockIdx.x / a.nsplit;
    const int split = (int)(blockIdx.x % a.nsplit);
    const int64_t bh = bhg / a.nqg, qg = bhg % a.nqg;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t hq0 = (h * a.nqg + qg) * NQ;   // first query head of this block
    const int64_t t_begin = (int64_t)split * a.split_len;
    const int64_t t_end = min(a.T, t_begin + a.split_len);

    float qv[NQ][8];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const float* p = a.qr + ((b * a.Hq + hq0 + qi) * D + 8 * li);
        const float4 x0 = *reinterpret_cast<const float4*>(p), x1 = *reinterpret_cast<const float4*>(p + 4);
        qv[qi][0] = x0.x; qv[qi][1] = x0.y; qv[qi][2] = x0.z; qv[qi][3] = x0.w;
        qv[qi][4] = x1.x; qv[qi][5] = x1.y; qv[qi][6] = x1.z; qv[qi][7] = x1.w;
    }
    float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        m[qi] = kNegBig;
        l[qi] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[qi][c] = 0.0f;
    }
    const uint8_t* kc = a.k_codes + bh * a.T * (D / 2) + 4 * li;
    const uint8_t* vc = a.v_codes + bh * a.T * (D / 2) + 4 * li;
    const int grp = (8 * li) / GS;
    const uint16_t* ksp = a.k_scale + bh * a.T * NGD + grp;
    const uint16_t* kzp = a.k_zero + bh * a.T * NGD + grp;
    const uint16_t* vsp = a.v_scale + bh * a.T * NGD + grp;
    const uint16_t* vzp = a.v_zero + bh * a.T * NGD + grp;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += TPS) {
        const int64_t t = t0 + wv * TPW + tg;
        const bool valid = t < t_end;
        const int64_t tc = valid ? t : t_end - 1;   // loads stay in the split
        const uint32_t wk = *reinterpret_cast<const uint32_t*>(kc + tc * (D / 2));
        const uint32_t wvv = *reinterpret_cast<const uint32_t*>(vc + tc * (D / 2));
        const float sk = bf_to_f(ksp[tc * NGD]), zk = -bf_to_f(kzp[tc * NGD]) * sk;
        const float sv = bf_to_f(vsp[tc * NGD]), zv = -bf_to_f(vzp[tc * NGD]) * sv;
        float kx[8], vx[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            kx[c] = __builtin_fmaf((float)((wk >> (4 * c)) & 15u), sk, zk);
            vx[c] = __builtin_fmaf((float)((wvv >> (4 * c)) & 15u), sv, zv);
        }
        float logit[NQ];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            float p = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) p = __builtin_fmaf(qv[qi][c], kx[c], p);
            logit[qi] = p;
        }
#pragma unroll
        for (int off = 1; off < LPT; off *= 2)
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) logit[qi] += __shfl_xor(logit[qi], off);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (valid && logit[qi] > m[qi]) {
                const float alpha = exp2f(m[qi] - logit[qi]);
                l[qi] *= alpha;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[qi][c] *= alpha;
                m[qi] = logit[qi];
            }
            const float p = valid ? exp2f(logit[qi] - m[qi]) : 0.0f;
            l[qi] += p;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[qi][c] = __builtin_fmaf(p, vx[c], acc[qi][c]);
        }
    }
    // merge the token groups of the wave, then the waves
#pragma unroll
    for (int off = LPT; off < 64; off *= 2) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const float mo = __shfl_xor(m[qi], off), lo = __shfl_xor(l[qi], off);
            const float M = fmaxf(m[qi], mo);
            const float sa = exp2f(m[qi] - M), sbb = exp2f(mo - M);
            l[qi] = l[qi] * sa + lo * sbb;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float ao = __shfl_xor(acc[qi][c], off);
                acc[qi][c] = acc[qi][c] * sa + ao * sbb;
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
        float* dst = a.part + ((b * a.Hq + hq0 + qi) * a.nsplit + split) * (D + 2);
        if (c == 0) { dst[0] = M; dst[1] = L; }
        dst[2 + c] = A;
    }
}

// Log-sum-exp merge of the splits of one (b, hq) row per wave, then the inverse rotation of the
// row: lane holds coordinates lane + 64 j, so stages 1 .. 32 run across lanes and 64, 128 inside.
template <int D, int OT>
__global__ void __launch_bounds__(256) rot_combine_kernel(const RotAttnArgs a, SignBits vs) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x % 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
    if (row >= a.B * a.Hq) return;   // uniform per wave
    const float* base = a.part + row * a.nsplit * (D + 2);
    float M = kNegBig;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, base[(int64_t)s * (D + 2)]);
    float L = 0.0f, A[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) A[j] = 0.0f;
    for (int s = 0; s < a.nsplit; ++s) {
        const float* sp = base + (int64_t)s * (D + 2);
        const float f = exp2f(sp[0] - M);
        L = __builtin_fmaf(sp[1], f, L);
#pragma unroll
        for (int j = 0; j < CPL; ++j) A[j] = __builtin_fmaf(sp[2 + lane + 64 * j], f, A[j]);
    }
    float v[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) v[j] = A[j] / L;
#pragma unroll
    for (int m = 1; m < 64 && m < D; m *= 2) {
        const bool hi = (lane & m) != 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const float p = __shfl_xor(v[j], m);
            v[j] = hi ? (p - v[j]) : (v[j] + p);
        }
    }
#pragma unroll
    for (int hj = 1; hj < CPL; hj *= 2) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if (j & hj) continue;
            const float x = v[j], y = v[j + hj];
            v[j] = x + y;
            v[j + hj] = x - y;
        }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        float x = v[j] * a.c;
        if ((sign8(vs, c & ~7) >> (c % 8)) & 1u) x = -x;
        if constexpr (OT == KVQ_FP32)
            static_cast<float*>(a.out)[row * D + c] = x;
        else
            static_cast<uint16_t*>(a.out)[row * D + c] = f_to_bf(x);
    }
}

template <int D, int G>
void launch_rot_quant(const void* K, const void* V, const RotGeom& geo, const SignBits& ks, const SignBits& vs,
                      const kvq_rot_cache& c, hipStream_t st) {
    const unsigned nblk = (unsigned)(geo.B * geo.ntt * geo.H);
    hipLaunchKernelGGL((rot_quant_kernel<D, G>), dim3(nblk), dim3(kThreads), 0, st, static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), geo, ks, vs, c);
}

template <int D, int G>
void launch_rot_dequant(const kvq_rot_cache& c, int side, const RotGeom& geo, const SignBits& sg, void* out, int ot,
                        hipStream_t st) {
    const unsigned nblk = (unsigned)(geo.B * geo.ntt * geo.H);
    const uint8_t* codes = side ? c.v_codes : c.k_codes;
    const uint16_t* sc = side ? c.v_scale : c.k_scale;
    const uint16_t* zr = side ? c.v_zero : c.k_zero;
    if (ot == KVQ_FP32)
        hipLaunchKernelGGL((rot_dequant_kernel<D, G, KVQ_FP32>), dim3(nblk), dim3(kThreads), 0, st, codes, sc, zr, geo,
                           sg, out);
    else
        hipLaunchKernelGGL((rot_dequant_kernel<D, G, KVQ_BF16>), dim3(nblk), dim3(kThreads), 0, st, codes, sc, zr, geo,
                           sg, out);
}

template <int D, int G>
void launch_rot_attn(const RotAttnArgs& a, int nq, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H * a.nqg * a.nsplit)), blk(kThreads);
    switch (nq) {   // heads per block: nq / nqg
        case 1: hipLaunchKernelGGL((rot_attn_split_kernel<D, G, 1>), grid, blk, 0, st, a); break;
        case 2: hipLaunchKernelGGL((rot_attn_split_kernel<D, G, 2>), grid, blk, 0, st, a); break;
        case 4: hipLaunchKernelGGL((rot_attn_split_kernel<D, G, 4>), grid, blk, 0, st, a); break;
        default: hipLaunchKernelGGL((rot_attn_split_kernel<D, G, 8>), grid, blk, 0, st, a); break;
    }
}

template <int D>
void launch_rot_q_combine(const RotAttnArgs& a, const SignBits& ks, const SignBits& vs, int ot, bool combine,
                          hipStream_t st) {
    if (!combine) {
        constexpr int RPP = kThreads / (D / 8);
        hipLaunchKernelGGL((rot_q_kernel<D>), dim3((unsigned)cdiv(a.B * a.Hq, RPP)), dim3(kThreads), 0, st, a, ks);
        return;
    }
    const dim3 grid((unsigned)cdiv(a.B * a.Hq, 4)), blk(256);
    if (ot == KVQ_FP32)
        hipLaunchKernelGGL((rot_combine_kernel<D, KVQ_FP32>), grid, blk, 0, st, a, vs);
    else
        hipLaunchKernelGGL((rot_combine_kernel<D, KVQ_BF16>), grid, blk, 0, st, a, vs);
}

int signs_of(const int8_t* s, int64_t d, SignBits& out, const char* name) {
    KVQ_REQUIRE(s, "%s: NULL signs", name);
    for (int i = 0; i < 8; ++i) out.w[i] = 0;
    for (int64_t c = 0; c < d; ++c) {
        KVQ_REQUIRE(s[c] == 1 || s[c] == -1, "%s: signs must be +1 or -1 (entry %lld is %d)", name, (long long)c,
                    (int)s[c]);
        if (s[c] < 0) out.w[c / 32] |= 1u << (c % 32);
    }
    return KVQ_OK;
}

int check_rot(const kvq_rot_cache* c, const char* name) {
    KVQ_REQUIRE(c, "%s: NULL cache descriptor", name);
    KVQ_REQUIRE(c->B >= 1 && c->T >= 1 && c->H >= 1, "%s: B, T, H must be >= 1", name);
    KVQ_REQUIRE(c->d == 64 || c->d == 128 || c->d == 256, "%s: d must be 64, 128 or 256", name);
    KVQ_REQUIRE((c->g == 32 || c->g == 64 || c->g == 128) && c->g <= c->d, "%s: g must be 32, 64 or 128 and <= d",
                name);
    KVQ_REQUIRE(c->B * c->T * c->H < ((int64_t)1 << 31), "%s: B * T * H must be below 2^31", name);
    const void* p[6] = {c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero};
    const char* nm[6] = {"k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"};
    for (int i = 0; i < 6; ++i) {
        KVQ_REQUIRE(p[i], "%s: NULL %s", name, nm[i]);
        KVQ_REQUIRE_ALIGNED(p[i], nm[i]);
    }
    return KVQ_OK;
}

RotGeom geom(const kvq_rot_cache* c) {
    RotGeom g;
    g.B = c->B; g.T = c->T; g.H = c->H;
    g.c = (float)(1.0 / std::sqrt((double)c->d));
    g.rows = (uint32_t)(c->B * c->T * c->H);
    g.ntt = (uint32_t)cdiv(c->T, kRowsPerBlock);
    return g;
}

// Token splits: about 1024 blocks in all; at d = 128 the matrix-core kernel takes the splits
// (multiples of 512 tokens, so every wave's range starts on a 128-token boundary), otherwise the
// VALU kernel (multiples of 64).
bool rot_mfma(const kvq_rot_cache* c) { return c->d == 128; }
int64_t rot_split_len(const kvq_rot_cache* c) {
    const int64_t want = cdiv(1024, c->B * c->H), unit = rot_mfma(c) ? 512 : 64;
    int64_t len = cdiv(cdiv(c->T, want), unit) * unit;
    return len < unit ? unit : len;
}

}  // namespace
}  // namespace kvq

extern "C" {

int kvq_rot_cache_sizes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, size_t sect_bytes[6], size_t* total) {
    KVQ_REQUIRE(sect_bytes && total, "kvq_rot_cache_sizes: NULL output");
    KVQ_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 2 && d % 2 == 0 && g >= 1 && d % g == 0,
                "kvq_rot_cache_sizes: invalid shape");
    const size_t n = (size_t)(B * H * T);
    sect_bytes[0] = sect_bytes[3] = n * (size_t)(d / 2);
    sect_bytes[1] = sect_bytes[2] = sect_bytes[4] = sect_bytes[5] = n * (size_t)(d / g) * 2;
    *total = 0;
    for (int i = 0; i < 6; ++i) *total += sect_bytes[i];
    return KVQ_OK;
}

int kvq_rot_quant_int4(const void* K, const void* V, const int8_t* k_signs, const int8_t* v_signs,
                       const kvq_rot_cache* c, kvq_stream stream) {
    int rc = kvq::check_rot(c, "kvq_rot_quant_int4");
    if (rc) return rc;
    KVQ_REQUIRE(K && V, "kvq_rot_quant_int4: NULL K or V");
    KVQ_REQUIRE_ALIGNED(K, "K");
    KVQ_REQUIRE_ALIGNED(V, "V");
    kvq::SignBits ks, vs;
    if ((rc = kvq::signs_of(k_signs, c->d, ks, "kvq_rot_quant_int4 (k_signs)"))) return rc;
    if ((rc = kvq::signs_of(v_signs, c->d, vs, "kvq_rot_quant_int4 (v_signs)"))) return rc;
    const kvq::RotGeom geo = kvq::geom(c);
    KVQ_DISPATCH_DG(c->d, c->g, kvq::launch_rot_quant, K, V, geo, ks, vs, *c, static_cast<hipStream_t>(stream));
    return kvq::launch_status("kvq_rot_quant_int4");
}

int kvq_rot_dequant(const kvq_rot_cache* c, int side, const int8_t* signs, void* out, int ot, kvq_stream stream) {
    int rc = kvq::check_rot(c, "kvq_rot_dequant");
    if (rc) return rc;
    KVQ_REQUIRE(side == 0 || side == 1, "kvq_rot_dequant: side must be 0 (K) or 1 (V)");
    KVQ_REQUIRE(out, "kvq_rot_dequant: NULL out");
    KVQ_REQUIRE(ot == KVQ_FP32 || ot == KVQ_BF16, "kvq_rot_dequant: ot must be KVQ_FP32 or KVQ_BF16");
    KVQ_REQUIRE_ALIGNED(out, "out");
    kvq::SignBits sg;
    if ((rc = kvq::signs_of(signs, c->d, sg, "kvq_rot_dequant"))) return rc;
    const kvq::RotGeom geo = kvq::geom(c);
    KVQ_DISPATCH_DG(c->d, c->g, kvq::launch_rot_dequant, *c, side, geo, sg, out, ot, static_cast<hipStream_t>(stream));
    return kvq::launch_status("kvq_rot_dequant");
}

size_t kvq_rot_decode_attn_ws(const kvq_rot_cache* c, int64_t Hq) {
    if (!c || c->B < 1 || c->T < 1 || c->H < 1 || c->d < 1 || Hq < 1) return 0;
    const int64_t nsplit = kvq::cdiv(c->T, kvq::rot_split_len(c));
    const size_t q = (size_t)(c->B * Hq * c->d) * sizeof(float);
    return kvq::cdiv((int64_t)q, 256) * 256 + (size_t)(c->B * Hq * nsplit * (c->d + 2)) * sizeof(float);
}

int kvq_rot_decode_attn(const kvq_rot_cache* c, const int8_t* k_signs, const int8_t* v_signs, const void* q,
                        int64_t Hq, float sm_scale, void* out, int ot, void* ws, size_t ws_bytes, kvq_stream stream) {
    int rc = kvq::check_rot(c, "kvq_rot_decode_attn");
    if (rc) return rc;
    KVQ_REQUIRE(q && out, "kvq_rot_decode_attn: NULL q or out");
    KVQ_REQUIRE(ot == KVQ_FP32 || ot == KVQ_BF16, "kvq_rot_decode_attn: ot must be KVQ_FP32 or KVQ_BF16");
    KVQ_REQUIRE(Hq >= 1 && Hq % c->H == 0, "kvq_rot_decode_attn: Hq must be a multiple of H");
    const int64_t nq = Hq / c->H;
    KVQ_REQUIRE(nq == 1 || nq == 2 || nq == 4 || nq == 8 || nq == 16, "kvq_rot_decode_attn: Hq / H must be 1, 2, 4, 8 or 16");
    const size_t need = kvq_rot_decode_attn_ws(c, Hq);
    KVQ_REQUIRE(ws && ws_bytes >= need, "kvq_rot_decode_attn: workspace of %zu bytes needed", need);
    KVQ_REQUIRE_ALIGNED(q, "q");
    KVQ_REQUIRE_ALIGNED(out, "out");
    KVQ_REQUIRE_ALIGNED(ws, "ws");
    kvq::SignBits ks, vs;
    if ((rc = kvq::signs_of(k_signs, c->d, ks, "kvq_rot_decode_attn (k_signs)"))) return rc;
    if ((rc = kvq::signs_of(v_signs, c->d, vs, "kvq_rot_decode_attn (v_signs)"))) return rc;
    kvq::RotAttnArgs a;
    a.k_codes = c->k_codes; a.k_scale = c->k_scale; a.k_zero = c->k_zero;
    a.v_codes = c->v_codes; a.v_scale = c->v_scale; a.v_zero = c->v_zero;
    a.q = static_cast<const uint16_t*>(q);
    a.qr = static_cast<float*>(ws);
    a.part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                      kvq::cdiv((int64_t)(c->B * Hq * c->d * sizeof(float)), 256) * 256);
    a.out = out;
    a.B = c->B; a.T = c->T; a.H = c->H; a.Hq = Hq;
    a.split_len = kvq::rot_split_len(c);
    a.nsplit = (int)kvq::cdiv(c->T, a.split_len);
    a.nqg = nq > 8 ? (int)(nq / 8) : 1;
    a.c = (float)(1.0 / std::sqrt((double)c->d));
    a.qscale = sm_scale * 1.4426950408889634f;
    KVQ_REQUIRE(c->B * c->H * a.nqg * a.nsplit < ((int64_t)1 << 31), "kvq_rot_decode_attn: grid too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (c->d == 64) kvq::launch_rot_q_combine<64>(a, ks, vs, ot, false, st);
    else if (c->d == 128) kvq::launch_rot_q_combine<128>(a, ks, vs, ot, false, st);
    else kvq::launch_rot_q_combine<256>(a, ks, vs, ot, false, st);
    if (kvq::rot_mfma(c))
        kvq::launch_attn_mfma_rot(c, a.qr, Hq, a.part, a.nsplit, a.split_len, st);
    else
        KVQ_DISPATCH_DG(c->d, c->g, kvq::launch_rot_attn, a, (int)nq, st);
    if (c->d == 64) kvq::launch_rot_q_combine<64>(a, ks, vs, ot, true, st);
    else if (c->d == 128) kvq::launch_rot_q_combine<128>(a, ks, vs, ot, true, st);
    else kvq::launch_rot_q_combine<256>(a, ks, vs, ot, true, st);
    return kvq::launch_status("kvq_rot_decode_attn");
}

}  // extern "C"
