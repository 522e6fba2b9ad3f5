// attn_mfma.hip -- the INT4 part of GQA decode attention on the gfx950 matrix cores
// (Explainer (KV cache 压缩：把历史装得更小): the attention kernel reads the low-bit cache and
// dequantizes it; fusing the dequantization is what turns fewer bytes into bandwidth).
//
// Per (b, KV head h, token split) block of 4 waves; each wave streams 32-token tiles of its
// own contiguous token range and keeps an online softmax for the Hq/H query heads of h.
// Both products are v_mfma_f32_16x16x32_f16 (16 rows x 16 columns x 32-deep):
//
//   scores  S[t][n]  = sum_c code_K[t][c] * Q'[n][c],   Q' = q * s_K * log2(e) as fp16 hi + lo
//           logit    = S - bias[n],  bias[n] = sum_c Q'[n][c] * z_K[c]
//           (K scales and zeros are per channel over a token group, so they fold into Q'; Q' is
//           split into two fp16 parts, two MFMAs each, so it carries ~22 significant bits)
//   values  O[c][n] += sum_t code_V[t][c] * P'[t][n],            P' = p * s_V[t][grp(c)] (fp16)
//           O[c][n] -= sum_t P'[t][n] * z_V[t][grp(c)]
//           (V scales and zeros are per token per channel group, so they fold into P')
//
// Codes become fp16 without a convert instruction: (0x6400 | n) is fp16(1024 + n), so after
// masking nibbles into bytes one v_perm_b32 (against a register holding 0x64006400) yields two
// fp16(1024 + code) values, and one packed fp16 add of -1024 leaves the exact codes.
//
// Lane layouts (verified for this builtin): A[m][k] in lane m%16 + 16*(k/8), element k%8;
// B[k][n] in lane n + 16*(k/8), element k%8; D[m][n] in lane n + 16*(m/4), element m%4.
//   QK: A = K codes, m = token (16 per MFMA), k = channel; lane group G = lane/16 owns the 32
//       channels 32G..32G+31 (one 16-byte load), element j of chunk kk is channel
//       32G + 8kk + perm[j] with perm = 0,2,4,6,1,3,5,7 (the order the byte pairing yields);
//       B = Q'^T with the same channel order; D gives lane (n, G) the scores of tokens
//       4G..4G+3 and 16+4G..16+4G+3 for query n.
//   PV: B = P'^T straight from those registers (k = token slots in that same order, n = query);
//       A = V codes^T, m = channel row, k = token; channel row m of block nb is channel
//       g*(nb/BPG) + BPG*m + nb%BPG (BPG = g/16 blocks per V group), so each MFMA's 16
//       channels share one V group (one P') and a lane's channels are adjacent nibbles.
//       The V code tile is staged through LDS to transpose tokens into the k dimension.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTile = 32;           // tokens per wave iteration
constexpr int D = 128;
constexpr float kNegBig = -3.0e38f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct MfmaArgs {
    const uint8_t* k_codes;
    const uint16_t* k_scale;
    const uint16_t* k_zero;
    const uint8_t* v_codes;
    const uint16_t* v_scale;
    const uint16_t* v_zero;
    const uint16_t* q;
    float* ws;
    int64_t B, H, Tq, nKg, Hq;
    int64_t split_len;   // tokens per split (multiple of 4 * kTile and of g)
    int nsplit;          // INT4 splits per (b, h)
    int nslot;           // partial slots per (b, hq) in ws (INT4 splits + residual splits)
    float qscale;        // sm_scale * log2(e)
};

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    half2v h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// two fp16(1024 + n) -> two exact fp16(n)
__device__ __forceinline__ uint32_t sub1024(uint32_t w) {
    const half2v off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, w) + off);
}

// Byte select that places a 0x64 exponent byte above each selected nibble byte: with
// c64 = 0x64006400 as the high source, perm(c64, x, sel) builds fp16(1024 + x.byte) pairs.
__device__ __forceinline__ uint32_t perm64(uint32_t x, uint32_t c64, uint32_t sel) {
    return __builtin_amdgcn_perm(c64, x, sel);
}
constexpr uint32_t kSelB0B1 = 0x07010500u;   // bytes 0, 1 of x -> fp16 pair
constexpr uint32_t kSelB2B3 = 0x07030502u;   // bytes 2, 3 of x
constexpr uint32_t kSelB0B2 = 0x07020500u;   // bytes 0, 2
constexpr uint32_t kSelB1B3 = 0x07030501u;   // bytes 1, 3

// 8 nibbles of a dword (byte j = c(2j) | c(2j+1) << 4) -> fp16(code) in the order
// c0,c2,c4,c6,c1,c3,c5,c7: mask the low and high nibbles into bytes, then pair bytes.
__device__ __forceinline__ half8 nib8(uint32_t w, uint32_t c64) {
    const uint32_t e = w & 0x0f0f0f0fu, o = (w >> 4) & 0x0f0f0f0fu;
    return as_half8(sub1024(perm64(e, c64, kSelB0B1)), sub1024(perm64(e, c64, kSelB2B3)),
                    sub1024(perm64(o, c64, kSelB0B1)), sub1024(perm64(o, c64, kSelB2B3)));
}

template <int GS, int NQ>
__global__ void __launch_bounds__(kThreads) attn_mfma_kernel(const MfmaArgs a) {
    constexpr int NG = D / GS;          // V groups per token
    constexpr int BPG = GS / 16;        // MFMA channel blocks per V group
    constexpr int PB = GS / 32;         // bytes of one V group piece per lane per token
    static_assert(NQ <= 16, "at most 16 query heads per KV head");

    // per-wave V code tile (32 tokens x 64 bytes) and its scales/zeros; reused for the merge
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kWaves][kTile * D / 2];
    __shared__ __attribute__((aligned(16))) uint16_t s_vs[kWaves][kTile * NG];
    __shared__ __attribute__((aligned(16))) uint16_t s_vz[kWaves][kTile * NG];
    __shared__ __attribute__((aligned(16))) uint16_t s_kp[kWaves][2 * D];   // K group scale, zero
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];
    __shared__ float s_o[kWaves][16][D + 1];

    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int n = lane % 16, G = lane / 16;
    const int64_t bh = blockIdx.x / a.nsplit;
    const int split = (int)(blockIdx.x % a.nsplit);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t Tq = a.Tq;
    // this wave's contiguous token range inside the split
    const int64_t s_lo = (int64_t)split * a.split_len;
    const int64_t s_hi = min(Tq, s_lo + a.split_len);
    const int64_t per_wave = a.split_len / kWaves;
    const int64_t t_lo = min(s_hi, s_lo + per_wave * wv);
    const int64_t t_hi = min(s_hi, t_lo + per_wave);

    // query n, channels 32G..32G+31 (zero for padding columns n >= NQ); sm_scale * log2(e) is
    // applied to the finished logits
    float qv[32];
    {
        const bool real = n < NQ;
        const uint16_t* qp = a.q + ((b * a.Hq + h * NQ + (real ? n : 0)) * D + 32 * G);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint4 r = *reinterpret_cast<const uint4*>(qp + 8 * u);
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qv[8 * u + 2 * e] = real ? bf_lo(w[e]) : 0.0f;
                qv[8 * u + 2 * e + 1] = real ? bf_hi(w[e]) : 0.0f;
            }
        }
    }
    const uint32_t c64 = 0x64006400u;

    floatx4 acc_o[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc_o[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = kNegBig, l_part = 0.0f;
    float zterm[NG];
#pragma unroll
    for (int gI = 0; gI < NG; ++gI) zterm[gI] = 0.0f;

    half8 bq[4], bql[4];   // Q'^T operand of the current K group: fp16 hi and lo parts
    float bias = 0.0f;

    const uint8_t* kc = a.k_codes + (b * a.H + h) * Tq * (D / 2);
    const uint8_t* vc = a.v_codes + (b * a.H + h) * Tq * (D / 2);
    const uint16_t* vsp = a.v_scale + (b * a.H + h) * Tq * NG;
    const uint16_t* vzp = a.v_zero + (b * a.H + h) * Tq * NG;
    const uint16_t* kscale = a.k_scale + (b * a.H + h) * a.nKg * D;
    const uint16_t* kzero = a.k_zero + (b * a.H + h) * a.nKg * D;
    uint8_t* sv = s_v[wv];

    // ---- one tile of global loads, issued one tile ahead of its use ----
    // K codes: token 16*hf + n, bytes 16G..16G+15.  V codes: 16-byte unit lane + 64j of the
    // 2 KB tile.  V scale/zero: one dword (two bf16) for lanes < 32*NG/2.  K group scale/zero:
    // lanes 0..15 the scale row, 16..31 the zero row (16 bytes each), when the tile opens a group.
    uint4 kr[2], vr[2], kp = make_uint4(0u, 0u, 0u, 0u);
    uint32_t vs2 = 0u, vz2 = 0u;
    auto fetch = [&](int64_t tt0) {
        const int nv = (int)min<int64_t>(kTile, t_hi - tt0);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int tt = min(16 * hf + n, nv - 1);
            kr[hf] = *reinterpret_cast<const uint4*>(kc + (tt0 + tt) * (D / 2) + 16 * G);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int u = lane + 64 * j;
            const int row = min(u / 4, nv - 1);
            vr[j] = *reinterpret_cast<const uint4*>(vc + (tt0 + row) * (D / 2) + 16 * (u % 4));
        }
        if (lane < kTile * NG / 2) {
            const int e0 = 2 * lane;
            const int row = min(e0 / NG, nv - 1);
            const int64_t off = (tt0 + row) * NG + e0 % NG;
            if (NG == 1) {
                const int row1 = min(e0 + 1, nv - 1);
                vs2 = (uint32_t)vsp[off] | ((uint32_t)vsp[tt0 + row1] << 16);
                vz2 = (uint32_t)vzp[off] | ((uint32_t)vzp[tt0 + row1] << 16);
            } else {
                vs2 = *reinterpret_cast<const uint32_t*>(vsp + off);
                vz2 = *reinterpret_cast<const uint32_t*>(vzp + off);
            }
        }
        if ((tt0 % GS == 0 || tt0 == t_lo) && lane < 32) {
            const uint16_t* src = (lane < 16 ? kscale : kzero) + (tt0 / GS) * D + 8 * (lane % 16);
            kp = *reinterpret_cast<const uint4*>(src);
        }
    };
    if (t_lo < t_hi) fetch(t_lo);

    for (int64_t t0 = t_lo; t0 < t_hi; t0 += kTile) {
        const int nvalid = (int)min<int64_t>(kTile, t_hi - t0);
        const bool new_grp = (t0 % GS == 0) || (t0 == t_lo);
        // ---- stage this tile (V codes, V params, K group params) in LDS; keep K codes ----
        *reinterpret_cast<uint4*>(sv + 16 * lane) = vr[0];
        *reinterpret_cast<uint4*>(sv + 16 * (lane + 64)) = vr[1];
        if (lane < kTile * NG / 2) {
            reinterpret_cast<uint32_t*>(s_vs[wv])[lane] = vs2;
            reinterpret_cast<uint32_t*>(s_vz[wv])[lane] = vz2;
        }
        if (new_grp && lane < 32) reinterpret_cast<uint4*>(s_kp[wv])[lane] = kp;
        const uint4 kcur0 = kr[0], kcur1 = kr[1];
        if (t0 + kTile < t_hi) fetch(t0 + kTile);
        __builtin_amdgcn_wave_barrier();

        // ---- K group parameters -> Q'^T operand (fp16 hi + lo) and bias ----
        if (new_grp) {
            constexpr int perm[8] = {0, 2, 4, 6, 1, 3, 5, 7};
            const uint32_t* ksw = reinterpret_cast<const uint32_t*>(s_kp[wv]) + 16 * G;        // scale, 32 bf16
            const uint32_t* kzw = reinterpret_cast<const uint32_t*>(s_kp[wv]) + 64 + 16 * G;   // zero, 32 bf16
            float bpart = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                uint32_t w[4], wl[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c0 = 8 * kk + perm[2 * e], c1 = 8 * kk + perm[2 * e + 1];
                    const uint32_t sw0 = ksw[c0 / 2], sw1 = ksw[c1 / 2], zw0 = kzw[c0 / 2], zw1 = kzw[c1 / 2];
                    const float s0 = (c0 & 1) ? bf_hi(sw0) : bf_lo(sw0), s1 = (c1 & 1) ? bf_hi(sw1) : bf_lo(sw1);
                    const float z0 = (c0 & 1) ? bf_hi(zw0) : bf_lo(zw0), z1 = (c1 & 1) ? bf_hi(zw1) : bf_lo(zw1);
                    const float q0 = qv[c0] * s0, q1 = qv[c1] * s1;
                    w[e] = pack_h2(q0, q1);
                    const half2v hq = __builtin_bit_cast(half2v, w[e]);
                    wl[e] = pack_h2(q0 - (float)hq[0], q1 - (float)hq[1]);
                    bpart = __builtin_fmaf(q0, z0, bpart);
                    bpart = __builtin_fmaf(q1, z1, bpart);
                }
                bq[kk] = as_half8(w[0], w[1], w[2], w[3]);
                bql[kk] = as_half8(wl[0], wl[1], wl[2], wl[3]);
            }
            bpart += __shfl_xor(bpart, 16);
            bpart += __shfl_xor(bpart, 32);
            bias = bpart;
        }

        // ---- scores ----
        floatx4 sc[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint4 kraw = hf ? kcur1 : kcur0;
            const uint32_t kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
            floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const half8 ak = nib8(kw[kk], c64);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bq[kk], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bql[kk], c, 0, 0, 0);
            }
            sc[hf] = c;
        }
        // lane (n, G): tokens 4G+i (half 0) and 16+4G+i (half 1), i = 0..3
        float lg[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lg[i] = (sc[0][i] - bias) * a.qscale;
            lg[4 + i] = (sc[1][i] - bias) * a.qscale;
        }
        if (nvalid < kTile) {   // only the last tile of a range is partial
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * G + i >= nvalid) lg[i] = kNegBig;
                if (16 + 4 * G + i >= nvalid) lg[4 + i] = kNegBig;
            }
        }
        float tmax = vmax3(vmax3(lg[0], lg[1], lg[2]), vmax3(lg[3], lg[4], lg[5]), vmax2(lg[6], lg[7]));
        tmax = vmax2(tmax, __shfl_xor(tmax, 16));
        tmax = vmax2(tmax, __shfl_xor(tmax, 32));
        const float m_new = vmax2(m_run, tmax);
        if (__any(m_new != m_run)) {          // rescale only when some running max moved
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_part *= alpha;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) acc_o[nb] *= alpha;
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) zterm[gI] *= alpha;
            m_run = m_new;
        }
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(lg[i] - m_run);
            l_part += p[i];
        }

        // ---- P' = p * s_V per V group (fp16), and the zero-point term ----
        half8 bp[NG];
        {
            // scales / zeros of tokens 4G..4G+3 and 16+4G..16+4G+3: 4*NG contiguous bf16 each
            uint32_t sv4[2][2 * NG], zv4[2][2 * NG];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int t4 = 16 * hf + 4 * G;
#pragma unroll
                for (int e = 0; e < 2 * NG; ++e) {
                    sv4[hf][e] = reinterpret_cast<const uint32_t*>(s_vs[wv] + t4 * NG)[e];
                    zv4[hf][e] = reinterpret_cast<const uint32_t*>(s_vz[wv] + t4 * NG)[e];
                }
            }
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // token slots 2e, 2e+1 -> half hf = e / 2, tokens i = 2(e%2), 2(e%2)+1 of that half
                    const int hf = e / 2, i0 = 2 * (e % 2), i1 = i0 + 1;
                    const int x0 = i0 * NG + gI, x1 = i1 * NG + gI;   // bf16 index within the 4-token run
                    const float sa = (x0 & 1) ? bf_hi(sv4[hf][x0 / 2]) : bf_lo(sv4[hf][x0 / 2]);
                    const float sb = (x1 & 1) ? bf_hi(sv4[hf][x1 / 2]) : bf_lo(sv4[hf][x1 / 2]);
                    const float za = (x0 & 1) ? bf_hi(zv4[hf][x0 / 2]) : bf_lo(zv4[hf][x0 / 2]);
                    const float zb = (x1 & 1) ? bf_hi(zv4[hf][x1 / 2]) : bf_lo(zv4[hf][x1 / 2]);
                    w[e] = pack_h2(p[2 * e] * sa, p[2 * e + 1] * sb);
                    const half2v hp = __builtin_bit_cast(half2v, w[e]);
                    zterm[gI] = __builtin_fmaf((float)hp[0], za, zterm[gI]);
                    zterm[gI] = __builtin_fmaf((float)hp[1], zb, zterm[gI]);
                }
                bp[gI] = as_half8(w[0], w[1], w[2], w[3]);
            }
        }

        // ---- values: transpose the code tile through LDS, 8 MFMAs ----
        {
            const int tok[8] = {4 * G, 4 * G + 1, 4 * G + 2, 4 * G + 3,
                                16 + 4 * G, 16 + 4 * G + 1, 16 + 4 * G + 2, 16 + 4 * G + 3};
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) {
                // this lane's piece of group gI: PB bytes at byte offset (GS/2)*gI + PB*n
                const int boff = (GS / 2) * gI + PB * n;
                const uint32_t o = (uint32_t)(boff & 3);
                uint32_t wd[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) wd[j] = *reinterpret_cast<const uint32_t*>(sv + tok[j] * (D / 2) + (boff & ~3));
                // dword per token pair: the pair's pieces side by side (token a low, token b high)
                uint32_t P[4][2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (PB == 1) {
                        P[e][0] = __builtin_amdgcn_perm(wd[2 * e + 1], wd[2 * e], o | ((4u + o) << 8));   // [a, b]
                    } else if constexpr (PB == 2) {
                        P[e][0] = __builtin_amdgcn_perm(wd[2 * e + 1], wd[2 * e], o | ((o + 1u) << 8) | ((4u + o) << 16) | ((5u + o) << 24));
                    } else {
                        P[e][0] = __builtin_amdgcn_perm(wd[2 * e + 1], wd[2 * e], 0x05040100u);
                        P[e][1] = __builtin_amdgcn_perm(wd[2 * e + 1], wd[2 * e], 0x07060302u);
                    }
                }
                // nibble k of both tokens -> fp16 pair: mask nibbles into bytes, pair the bytes
#pragma unroll
                for (int k = 0; k < BPG; ++k) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t src = P[e][k / 4];
                        const uint32_t nib = (k & 1) ? ((src >> 4) & 0x0f0f0f0fu) : (src & 0x0f0f0f0fu);
                        uint32_t sel;
                        if constexpr (PB == 1) sel = kSelB0B1;                                // bytes [a, b]
                        else sel = ((k % 4) / 2) ? kSelB1B3 : kSelB0B2;                      // [a0 a1 b0 b1]
                        w[e] = sub1024(perm64(nib, c64, sel));
                    }
                    const int nb = gI * BPG + k;
                    acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(w[0], w[1], w[2], w[3]), bp[gI],
                                                                       acc_o[nb], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();     // LDS reads done before the next tile overwrites
    }

    // ---------------- finish the wave: sums over the 4 lane groups, zero-point term ----------------
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
#pragma unroll
    for (int gI = 0; gI < NG; ++gI) {
        zterm[gI] += __shfl_xor(zterm[gI], 16);
        zterm[gI] += __shfl_xor(zterm[gI], 32);
    }
    // acc_o[nb][i] is channel row m = 4G + i of block nb, query n
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int gI = nb / BPG, k = nb % BPG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * G + i;
            const int c = GS * gI + BPG * m + k;
            s_o[wv][n][c] = acc_o[nb][i] - zterm[gI];
        }
    }
    if (G == 0) { s_m[wv][n] = m_run; s_l[wv][n] = l_part; }
    __syncthreads();
    // merge the 4 waves and write (m, l, acc[D]) for each real query
    for (int e = tid; e < NQ * D; e += kThreads) {
        const int qn = e / D, c = e % D;
        float M = s_m[0][qn];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = vmax2(M, s_m[w][qn]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2f(s_m[w][qn] - M);
            L = __builtin_fmaf(s_l[w][qn], f, L);
            A = __builtin_fmaf(s_o[w][qn][c], f, A);
        }
        float* dst = a.ws + ((b * a.Hq + h * NQ + qn) * a.nslot + split) * (D + 2);
        if (c == 0) { dst[0] = M; dst[1] = L; }
        dst[2 + c] = A;
    }
}

template <int GS>
void launch_nq(const MfmaArgs& a, int nq, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H * a.nsplit)), blk(kThreads);
    switch (nq) {
        case 1: hipLaunchKernelGGL((attn_mfma_kernel<GS, 1>), grid, blk, 0, st, a); break;
        case 2: hipLaunchKernelGGL((attn_mfma_kernel<GS, 2>), grid, blk, 0, st, a); break;
        case 4: hipLaunchKernelGGL((attn_mfma_kernel<GS, 4>), grid, blk, 0, st, a); break;
        case 8: hipLaunchKernelGGL((attn_mfma_kernel<GS, 8>), grid, blk, 0, st, a); break;
        default: hipLaunchKernelGGL((attn_mfma_kernel<GS, 16>), grid, blk, 0, st, a); break;
    }
}

}  // namespace

// Launch the INT4 token range [0, Tq) on the matrix cores (d = 128).  Partials go to ws
// slots 0 .. nsplit-1 of each (b, hq); the caller owns slot counts and the combine.
void launch_attn_mfma(const kvq_int4_cache* c, const void* q, int64_t Hq, float qscale, float* ws, int nsplit,
                      int64_t split_len, int nslot, hipStream_t st) {
    MfmaArgs a;
    a.k_codes = c->k_codes; a.k_scale = c->k_scale; a.k_zero = c->k_zero;
    a.v_codes = c->v_codes; a.v_scale = c->v_scale; a.v_zero = c->v_zero;
    a.q = static_cast<const uint16_t*>(q);
    a.ws = ws;
    a.B = c->B; a.H = c->H; a.Tq = c->T - c->R; a.nKg = cdiv(a.Tq, c->g); a.Hq = Hq;
    a.split_len = split_len;
    a.nsplit = nsplit;
    a.nslot = nslot;
    a.qscale = qscale;
    const int nq = (int)(Hq / c->H);
    if (c->g == 32) launch_nq<32>(a, nq, st);
    else if (c->g == 64) launch_nq<64>(a, nq, st);
    else launch_nq<128>(a, nq, st);
}

}  // namespace kvq
