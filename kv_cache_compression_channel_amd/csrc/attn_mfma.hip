// attn_mfma.hip -- the INT4 part of GQA decode attention on the gfx950 matrix cores
// (Explainer (KV cache 压缩：把历史装得更小): the attention kernel reads the low-bit cache and
// dequantizes it; fusing the dequantization is what turns fewer bytes into bandwidth).
//
// Per (b, KV head h, token split) block of 4 waves; each wave streams 32-token tiles of its
// own contiguous token range and keeps an online softmax for the Hq/H query heads of h.
// Both products are v_mfma_f32_16x16x32_f16 (16 rows x 16 columns x 32-deep).
//
// Codes enter the matrix cores as fp16(64 + code): with 0x54 as the high byte and the nibble
// in mantissa bits 4..7, one v_and_or_b32 turns a pair of nibbles into a pair of fp16 values
// (no convert, no subtract).  The constant 64 is removed on the other side of each product:
//
//   scores  S'[t][n] = sum_c (64 + code_K[t][c]) * Q'[n][c],   Q' = q * s_K (fp16 hi + lo)
//           logit    = (S' - bias[n]) * lscale,   bias[n] = sum_c q'[n][c] * (z_K[c] + 64)
//           (K scales and zeros are per channel over a token group, so they fold into Q'; Q' is
//           split into two fp16 parts, two MFMAs each, so it carries ~22 significant bits; the
//           bias is formed in fp32 from the unrounded q')
//   values  O[c][n] = sum_t (64 + code_V[t][c]) * P'[t][n]  -  sum_t (64 + z_V[t][grp(c)]) * P'[t][n],
//                     P' = fp16(p * s_V)
//           (the second term is one more MFMA per V group, whose A operand holds fp16(64 + z_V)
//           of each token -- exact, as a stored zero point is an integer of magnitude <= 256 --
//           so both terms carry the same rounded weight and its rounding cancels inside
//           (code - z); the rotated cache keeps its own form of the zero-point term, see ROT)
//
// The fp16 range is kept by the softmax reference: p = 2^(logit - ref) with
// ref = Mlog + E - 15, where Mlog bounds every logit seen so far and 2^E bounds every V scale
// seen so far, so P' = p * s_V < 2^15.  The reference only moves (with the usual rescale of
// the running sums) when a tile holds a logit above Mlog or a scale at or above 2^E, which
// after the first tiles is rare; the partial it writes is (ref, l, O), which the log-sum-exp
// combine merges like any other.  A K group whose q * s_K would leave the fp16 range is
// scaled by a power of two per query, undone in lscale.
//
// Lane layouts (verified for this builtin): A[m][k] in lane m%16 + 16*(k/8), element k%8;
// B[k][n] in lane n + 16*(k/8), element k%8; D[m][n] in lane n + 16*(m/4), element m%4.
//   QK: A = K codes, m = token (16 per MFMA), k = channel; lane group G = lane/16 owns the 32
//       channels 32G..32G+31 (one 16-byte load), element j of chunk kk is channel
//       32G + 8kk + kPerm[j] (the order the nibble extraction yields); B = Q'^T in the same
//       channel order; D gives lane (n, G) the scores of tokens 4G..4G+3 and 16+4G..16+4G+3.
//   PV: B = P'^T straight from those registers (k = token slots in that same order, n = query);
//       A = V codes^T, m = channel row, k = token; channel row m of block nb is channel
//       g*(nb/BPG) + BPG*m + nb%BPG (BPG = g/16 blocks per V group), so each MFMA's 16
//       channels share one V group (one P') and a lane's channels are adjacent nibbles.
//       The V code tile is staged through LDS to bring tokens into the k dimension.
//   Q' for a new K group: with NQ query heads, lane (n, G) computes query n % NQ on 8-channel
//       chunk(s) of its 32 channels and the chunks are exchanged through LDS, so the work is
//       spread over all 16 lanes of a group instead of the NQ lanes that own real queries.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTile = 32;           // tokens per wave iteration
constexpr int D = 128;
constexpr float kNegBig = -3.0e38f;
constexpr float kMargin = 2.0f;     // head-room put above the largest logit when the reference moves
constexpr int kEmin = -64, kEmax = 64;
// Buffer resource word 3 for raw byte-addressed loads (32-bit data format, no swizzle or thread
// offset), and the non-temporal cache policy of a buffer load.
constexpr int kBufferFormat = 0x00020000;
constexpr int kLoadNT = 2;

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
    const uint16_t* k_res;
    const uint16_t* v_res;
    const uint16_t* q;
    const float* qrot;       // ROT mode: rotated queries [B][Hq][D] fp32, already times sm_scale * log2(e)
    float* ws;
    float* lgw;              // base-2 logits [B][Hq][ldl] (token t of head (b, hq) at row * ldl + t), or NULL
    int64_t ldl;
    int64_t B, H, Hq;
    int Tq, nKg;
    int64_t ldq, ldk, ldr;   // rows per (b, h) of the code / V-scale, K-group and residual sections
    int R;               // residual (bf16) tokens per (b, h)
    int nres;            // residual splits per (b, h), kResTile tokens each; their blocks come first
    int split_len;       // tokens per split (multiple of 4 * kTile)
    int nsplit;          // INT4 splits per (b, h)
    int nslot;           // partial slots per (b, hq) in ws: INT4 splits, then residual splits
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

// The fp16 pair (a - h.lo, b - h.hi) for h = pack_h2(a, b): each difference is exact in fp32 and
// v_fma_mix{lo,hi}_f16 (h's half taken as fp16, times -1, plus the fp32 value) round it once to
// fp16, which is what converting the fp32 difference gives -- in two instructions instead of five.
__device__ __forceinline__ uint32_t residual_h2(uint32_t h, float a, float b) {
    uint32_t r;   // the high half is written by the second instruction
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
    asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(h), "v"(b));
    return r;
}

// fp16 0x5400 | (n << 4) = 64 + n for a nibble n in mantissa bits 4..7.
constexpr uint32_t kMagic = 0x54005400u;
constexpr uint32_t kNib = 0x00f000f0u;
__device__ __forceinline__ uint32_t nib_pair(uint32_t x) {
    return __builtin_amdgcn_bitop3_b32(x, kNib, kMagic, 0xEA);   // (x & kNib) | kMagic in one op
}

// One dword of K codes (byte j = c(2j) | c(2j+1) << 4) -> fp16(64 + c) in the element order
// c0 c4 c2 c6 c1 c5 c3 c7: each pair takes the nibbles sitting in bits 4..7 and 20..23.
constexpr int kPerm[8] = {0, 4, 2, 6, 1, 5, 3, 7};
__device__ __forceinline__ half8 nib8(uint32_t w) {
    return as_half8(nib_pair(w << 4), nib_pair(w >> 4), nib_pair(w), nib_pair(w >> 8));
}

// ---- the bf16 residual window: one block per (b, h, split of up to kResTile tokens) ----
// Plain fp32 arithmetic from an LDS copy of the rows: logits q . k (q pre-scaled by
// sm_scale log2 e), base-2 softmax over the split, p-weighted sum of the V rows.  Writes the
// split's partial (max logit, sum of p, sum of p v) like every other split.
constexpr int kResTile = 64;
constexpr int kResPad = D + 8;      // row stride of the LDS copies (16-byte reads spread over the banks)
struct ResLds {
    uint16_t k[kResTile][kResPad];
    uint16_t v[kResTile][kResPad];
    float q[16][D];
    float p[16][kResTile];      // logits, then probabilities, per query
    float m[16], l[16];
};

template <int NQ, bool LG>
__device__ void residual_block(const MfmaArgs& a, ResLds& sr, int rb) {
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int64_t bh = rb / a.nres;
    const int split = rb % a.nres;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int r_lo = split * kResTile;
    const int nt = min(kResTile, a.R - r_lo);
    const uint16_t* kr = a.k_res + (bh * a.ldr + r_lo) * D;
    const uint16_t* vr = a.v_res + (bh * a.ldr + r_lo) * D;
    for (int i = tid; i < nt * (D / 8); i += kThreads) {
        const int t = i / (D / 8), c8 = 8 * (i % (D / 8));
        *reinterpret_cast<u32x4*>(&sr.k[t][c8]) = *reinterpret_cast<const u32x4*>(kr + t * D + c8);
        *reinterpret_cast<u32x4*>(&sr.v[t][c8]) = *reinterpret_cast<const u32x4*>(vr + t * D + c8);
    }
    const uint16_t* qp = a.q + (b * a.Hq + h * NQ) * D;
    for (int e = tid; e < NQ * D; e += kThreads) sr.q[e / D][e % D] = bf_to_f(qp[e]) * a.qscale;
    __syncthreads();
    // logits: token fastest across lanes, so a wave reads one query row (broadcast)
#pragma unroll 1
    for (int e = tid; e < nt * NQ; e += kThreads) {
        const int t = e % nt, n = e / nt;
        float acc = 0.0f;
#pragma unroll
        for (int j0 = 0; j0 < D / 8; j0 += 4) {   // a quarter of the row's loads in flight at once
          u32x4 kw[D / 8];
#pragma unroll
          for (int j = j0; j < j0 + 4; ++j) kw[j] = *reinterpret_cast<const u32x4*>(&sr.k[t][8 * j]);
#pragma unroll
          for (int j = j0; j < j0 + 4; ++j) {
            const float4 q0 = *reinterpret_cast<const float4*>(&sr.q[n][8 * j]);
            const float4 q1 = *reinterpret_cast<const float4*>(&sr.q[n][8 * j + 4]);
            acc = __builtin_fmaf(q0.x, bf_lo(kw[j][0]), acc);
            acc = __builtin_fmaf(q0.y, bf_hi(kw[j][0]), acc);
            acc = __builtin_fmaf(q0.z, bf_lo(kw[j][1]), acc);
            acc = __builtin_fmaf(q0.w, bf_hi(kw[j][1]), acc);
            acc = __builtin_fmaf(q1.x, bf_lo(kw[j][2]), acc);
            acc = __builtin_fmaf(q1.y, bf_hi(kw[j][2]), acc);
            acc = __builtin_fmaf(q1.z, bf_lo(kw[j][3]), acc);
            acc = __builtin_fmaf(q1.w, bf_hi(kw[j][3]), acc);
          }
        }
        sr.p[n][t] = acc;
        if constexpr (LG) a.lgw[(b * a.Hq + h * NQ + n) * a.ldl + a.Tq + r_lo + t] = acc;
    }
    __syncthreads();
    // softmax over the split: one wave per query, lanes over tokens
    for (int n = wv; n < NQ; n += kWaves) {
        const float x = lane < nt ? sr.p[n][lane] : kNegBig;
        const float m = max_lanes_desc<16>(max_halves(x));
        const float pv = lane < nt ? exp2f(x - m) : 0.0f;
        const float l = add_lanes_desc<16>(add_halves(pv));
        sr.p[n][lane] = pv;
        if (lane == 0) { sr.m[n] = m; sr.l[n] = l; }
    }
    __syncthreads();
    // partial output: channel pairs fastest across lanes, tokens in groups of 4
#pragma unroll 1
    for (int e = tid; e < NQ * (D / 2); e += kThreads) {
        const int n = e / (D / 2), c = 2 * (e % (D / 2));
        float a0 = 0.0f, a1 = 0.0f;
        int t = 0;
        for (; t + 4 <= nt; t += 4) {
            const float4 pw = *reinterpret_cast<const float4*>(&sr.p[n][t]);
            const uint32_t v0 = *reinterpret_cast<const uint32_t*>(&sr.v[t][c]);
            const uint32_t v1 = *reinterpret_cast<const uint32_t*>(&sr.v[t + 1][c]);
            const uint32_t v2 = *reinterpret_cast<const uint32_t*>(&sr.v[t + 2][c]);
            const uint32_t v3 = *reinterpret_cast<const uint32_t*>(&sr.v[t + 3][c]);
            a0 = __builtin_fmaf(pw.x, bf_lo(v0), a0); a1 = __builtin_fmaf(pw.x, bf_hi(v0), a1);
            a0 = __builtin_fmaf(pw.y, bf_lo(v1), a0); a1 = __builtin_fmaf(pw.y, bf_hi(v1), a1);
            a0 = __builtin_fmaf(pw.z, bf_lo(v2), a0); a1 = __builtin_fmaf(pw.z, bf_hi(v2), a1);
            a0 = __builtin_fmaf(pw.w, bf_lo(v3), a0); a1 = __builtin_fmaf(pw.w, bf_hi(v3), a1);
        }
        for (; t < nt; ++t) {
            const uint32_t v0 = *reinterpret_cast<const uint32_t*>(&sr.v[t][c]);
            a0 = __builtin_fmaf(sr.p[n][t], bf_lo(v0), a0);
            a1 = __builtin_fmaf(sr.p[n][t], bf_hi(v0), a1);
        }
        float* dst = a.ws + ((b * a.Hq + h * NQ + n) * a.nslot + (a.nslot - a.nres) + split) * (D + 2);
        if (c == 0) { dst[0] = sr.m[n]; dst[1] = sr.l[n]; }
        *reinterpret_cast<float2*>(dst + 2 + c) = make_float2(a0, a1);
    }
}

// Waves per SIMD the kernel is compiled for.  The plain KIVI kernel with at most 4 query heads
// per KV head and groups of 64 or 128 fits in 168 VGPRs without spilling, so 3 workgroups share a
// CU (47 KB of LDS each); the variants that also write logits, the rotated cache's and the
// others need more registers and run 2 per SIMD.
template <int GS, int NQ, bool LG, bool ROT>
constexpr int attn_waves() {
    return (!LG && !ROT && GS >= 64 && NQ <= 4) ? 3 : 2;
}

// ROT: the Hadamard-rotated per-token cache.  K is then grouped like V (a bf16 scale and zero per
// token and g channels), so the query needs no per-group scaling: Q' = q' (fp16 hi + lo, made
// once), each score MFMA covers 32 consecutive channels (one K group holds whole MFMAs), and
//   logit = sum_grp s_K[t][grp] * (S'_grp[t][n] - (64 + z_K[t][grp]) * sum_{c in grp} Q'[n][c]).
// The V side is the same as for the KIVI cache.
template <int GS, int NQ, bool LG, bool ROT = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(attn_waves<GS, NQ, LG, ROT>())))
attn_mfma_kernel(const MfmaArgs a) {
    constexpr int NG = D / GS;          // V groups per token
    constexpr int BPG = GS / 16;        // MFMA channel blocks per V group
    constexpr int PB = GS / 32;         // bytes of one V group piece per lane per token
    constexpr int PASS = NQ >= 16 ? 4 : (NQ == 8 ? 2 : 1);   // Q' chunks each lane computes
    static_assert(NQ <= 16, "at most 16 query heads per KV head");

    // per-wave V code tile (32 tokens x 64 bytes), V (scale, zero) pairs in fp32, K group
    // scale/zero rows, the Q' exchange; the merge at the end reuses the same memory
    struct Loop {
        uint8_t k[kWaves][2 * kTile * D / 2];   // the two tiles of a pair
        uint8_t v[kWaves][2 * kTile * D / 2];
        float sz[kWaves][2 * kTile * NG * 2];     // (scale, zero) of a tile pair
        uint16_t kp[kWaves][(GS == 32 ? 4 : 2) * D];   // K group scale and zero rows of a tile pair
        uint32_t qx[kWaves][ROT ? 1 : 64][PASS * 8];
        float ksz[kWaves][ROT ? 2 * kTile * NG * 2 : 1];   // ROT: K (scale, zero) of a tile pair
        uint16_t zf[kWaves][ROT ? 1 : 2 * NG * kTile];     // fp16(64 + z_V), [tile][group][token]
    };
    struct Merge {
        float m[kWaves][16], l[kWaves][16];
        float o[kWaves][16][D + 1];
    };
    __shared__ __attribute__((aligned(16))) union {
        Loop lp;
        Merge mg;
        ResLds rs;
    } sm;

    // Block order: the INT4 splits split-major (block = split * B*H + (b, h)), then the bf16
    // residual blocks.  Blocks go to the XCDs round-robin, so split-major order gives every XCD
    // the same share of the short last splits, and the residual blocks, dispatched last, take
    // the slots those splits free instead of delaying a long split at the start.
    const int nq_blocks = (int)(a.B * a.H) * a.nsplit;
    if ((int)blockIdx.x >= nq_blocks) {      // uniform per block
        residual_block<NQ, LG>(a, sm.rs, (int)blockIdx.x - nq_blocks);
        return;
    }
    const int blk = (int)blockIdx.x;

    const int tid = threadIdx.x, lane = tid % 64;
    const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
    const int n = lane % 16, G = lane / 16;
    const int64_t bh = blk % (a.B * a.H);
    const int split = (int)(blk / (a.B * a.H));
    const int64_t b = bh / a.H, h = bh % a.H;
    const int Tq = a.Tq;
    // this wave's contiguous token range inside the split
    const int s_lo = split * a.split_len;
    const int s_hi = min(Tq, s_lo + a.split_len);
    const int per_wave = a.split_len / kWaves;
    const int t_lo = min(s_hi, s_lo + per_wave * wv);
    const int t_hi = min(s_hi, t_lo + per_wave);

    // the query values this lane turns into Q': query n % NQ, channels 32G + 8 kc(p) + 0..7
    auto chunk_of = [&](int p) -> int {
        if constexpr (NQ >= 16) return p;
        else if constexpr (NQ == 8) return n / 8 + 2 * p;
        else return (n / NQ) % 4;
    };
    float qv[PASS][8];
    // ROT: Q'^T operands (fp16 hi, lo) of MFMA chunk kk = channels 32 kk + 8 G + kPerm[j], the
    // per-group sums of Q', and the power of two that keeps Q' inside the fp16 range
    u32x4 rq_hi[ROT ? 4 : 1], rq_lo[ROT ? 4 : 1];
    float rq_sum[ROT ? NG : 1];
    float rq_scale = 1.0f;
    if constexpr (ROT) {
        const float* qp = a.qrot + (b * a.Hq + h * NQ + n % NQ) * D;
        float x[4][8];
        float qmax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float4 x0 = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * G);
            const float4 x1 = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * G + 4);
            const float v8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[kk][j] = v8[kPerm[j]];
                qmax = vmax2(qmax, __builtin_fabsf(v8[j]));
            }
        }
        qmax = max_halves(vmax2(qmax, xor_lane<16>(qmax)));
        // |Q'| < 2^14 after the scaling (also for tiny queries, which are scaled up)
        const int tau = qmax > 0.0f ? __builtin_amdgcn_frexp_expf(qmax) - 14 : 0;
        rq_scale = __builtin_ldexpf(1.0f, tau);
        float csum[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint32_t hw[4], lw[4];
            float sum = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = __builtin_ldexpf(x[kk][2 * e], -tau), x1 = __builtin_ldexpf(x[kk][2 * e + 1], -tau);
                hw[e] = pack_h2(x0, x1);
                const half2v hh = __builtin_bit_cast(half2v, hw[e]);
                lw[e] = pack_h2(x0 - (float)hh[0], x1 - (float)hh[1]);
                const half2v ll = __builtin_bit_cast(half2v, lw[e]);
                sum += ((float)hh[0] + (float)ll[0]) + ((float)hh[1] + (float)ll[1]);
            }
            rq_hi[kk] = u32x4{hw[0], hw[1], hw[2], hw[3]};
            rq_lo[kk] = u32x4{lw[0], lw[1], lw[2], lw[3]};
            sum = add_halves(sum + xor_lane<16>(sum));
            csum[kk] = sum;      // the 32 channels of chunk kk, query n
        }
#pragma unroll
        for (int gI = 0; gI < NG; ++gI) {
            float t = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                if ((32 * kk) / GS == gI) t += csum[kk];
            rq_sum[gI] = t;
        }
    } else {
        const uint16_t* qp = a.q + (b * a.Hq + h * NQ + n % NQ) * D + 32 * G;
#pragma unroll
        for (int p = 0; p < PASS; ++p) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(qp + 8 * chunk_of(p));
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qv[p][2 * e] = bf_lo(w[e]);
                qv[p][2 * e + 1] = bf_hi(w[e]);
            }
        }
    }

    floatx4 acc_o[8], acc_off[NG];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc_o[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gI = 0; gI < NG; ++gI) acc_off[gI] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float zsum[NG];
#pragma unroll
    for (int gI = 0; gI < NG; ++gI) zsum[gI] = 0.0f;
    float l_part = 0.0f;
    // softmax reference (per query column) and its bounds
    float ref = 0.0f;            // p = 2^(logit - ref)
    float thr = kNegBig;         // largest logit - ref allowed without moving ref (= 15 - E once started)
    int e_s = kEmin;             // every V scale seen is below 2^e_s
    float s_lim = 0.0f;          // 2^e_s (0 before the first tile)
    bool started = false;

    float lscale = a.qscale, c0 = 0.0f;   // logit - ref = S' * lscale - c0

    const uint8_t* kc = a.k_codes + bh * a.ldq * (D / 2);
    const uint8_t* vc = a.v_codes + bh * a.ldq * (D / 2);
    const uint16_t* vsp = a.v_scale + bh * a.ldq * NG;
    const uint16_t* vzp = a.v_zero + bh * a.ldq * NG;
    const uint16_t* kscale = a.k_scale + bh * a.ldk * D;
    const uint16_t* kzero = a.k_zero + bh * a.ldk * D;
    uint8_t* sk = sm.lp.k[wv];
    uint8_t* sv = sm.lp.v[wv];
    float* ssz = sm.lp.sz[wv];
    uint16_t* skp = sm.lp.kp[wv];
    uint32_t* sqx = sm.lp.qx[wv][0];   // Q'^T chunks of the current K group (fp16 hi, lo) per lane

    // ---- tile loads: two tiles in flight per wave, in registers until staged ----
    // Tiles go in pairs (the wave's range starts on a 128-token boundary, so a pair never
    // straddles a K group of 64 or 128 tokens).  Every tile: K codes, token 16*hf + n, bytes
    // 16G..16G+15; V codes, 16-byte unit lane + 64j of the 2 KB tile.  The even tile of a pair
    // also brings the pair's side data in one access per array: the V (scale, zero) elements of
    // token lane of the pair, and the K group scale and zero rows (both groups of the pair when
    // g = 32: lane group G holds row G % 2 of the pair's group G / 2).
    // Every lane issues the same loads for every tile, whatever the position: rows past the
    // end of the cache read as zero (their logits are masked and their V scales are zero, so
    // they never count; the largest V scale of a pair is unchanged, as the pair holds the last
    // row).  With no load behind a branch, the wait before staging a tile leaves the loads of the
    // tile behind it in flight.
    constexpr int SW = NG >= 2 ? NG / 2 : 1;   // dwords of V scale (and of zero) per lane per pair
    struct CodeRegs {
        u32x4 k[2], v[2];
    };
    struct SideRegs {
        u32x4 kp;
        uint32_t vs[SW], vz[SW];
        uint32_t ks[SW], kz[SW];   // ROT: per-token K scale / zero, laid out like V's
    };
    const int last_row = Tq - 1;
    const uint16_t* kpsrc = (G % 2 ? kzero : kscale) + 8 * n;
    const uint16_t* kspt = a.k_scale + bh * a.ldq * NG;   // ROT: per-token K scale / zero rows
    const uint16_t* kzpt = a.k_zero + bh * a.ldq * NG;
    // Tile loads go through buffer resources that cover the rows [tt0, min(Tq, tt0 + n)) of a
    // section: a row at or past Tq reads as zero (a buffer load past the resource's size returns
    // zeros and touches no memory), so no lane clamps its row, and the lane offsets below stay
    // the same for every tile (the tile's position is in the resource, a scalar).
    auto rows_rsrc = [&](const void* base, int tt0, int nrow, int row_bytes) {
        const uint32_t size = (uint32_t)min(Tq - tt0, nrow) * (uint32_t)row_bytes;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)size, kBufferFormat);
    };
    const uint32_t off_k = (uint32_t)(n * (D / 2) + 16 * G);   // K: token n (+16), bytes 16G..16G+15
    const uint32_t off_v = (uint32_t)(16 * lane);              // V: 16-byte unit lane of the tile (+1 KB)
    auto fetch_codes = [&](CodeRegs& r, int tt0) {
        const auto rk = rows_rsrc(kc + (int64_t)tt0 * (D / 2), tt0, kTile, D / 2);
        const auto rv = rows_rsrc(vc + (int64_t)tt0 * (D / 2), tt0, kTile, D / 2);
        r.k[0] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_k, 0, kLoadNT);
        r.k[1] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_k + 16 * (D / 2), 0, kLoadNT);
        r.v[0] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_v, 0, kLoadNT);
        r.v[1] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_v + 16 * (D / 2), 0, kLoadNT);
    };
    // per-token (scale, zero) words of token lane of the pair: NG bf16 each (the (b, h) row of a
    // one-group-per-token section may be only 2-byte aligned, hence 2-byte loads for NG = 1)
    auto fetch_pt = [&](const uint16_t* sp, const uint16_t* zp, uint32_t (&os)[SW], uint32_t (&oz)[SW], int tt0) {
        const auto rs = rows_rsrc(sp + (int64_t)tt0 * NG, tt0, 2 * kTile, NG * 2);
        const auto rz = rows_rsrc(zp + (int64_t)tt0 * NG, tt0, 2 * kTile, NG * 2);
        const uint32_t e = (uint32_t)lane * (NG * 2);   // byte offset of token lane's elements
        if constexpr (NG == 1) {
            os[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, e, 0, kLoadNT);
            oz[0] = __builtin_amdgcn_raw_buffer_load_b16(rz, e, 0, kLoadNT);
        } else if constexpr (NG == 2) {
            os[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, e, 0, kLoadNT);
            oz[0] = __builtin_amdgcn_raw_buffer_load_b32(rz, e, 0, kLoadNT);
        } else {
            const auto a2 = __builtin_amdgcn_raw_buffer_load_b64(rs, e, 0, kLoadNT);
            const auto b2 = __builtin_amdgcn_raw_buffer_load_b64(rz, e, 0, kLoadNT);
            os[0] = a2[0]; os[1] = a2[1];
            oz[0] = b2[0]; oz[1] = b2[1];
        }
    };
    auto fetch_side = [&](SideRegs& r, int tt0) {
        fetch_pt(vsp, vzp, r.vs, r.vz, tt0);
        if constexpr (ROT) {
            fetch_pt(kspt, kzpt, r.ks, r.kz, tt0);
        } else {
            const int gt = GS == 32 ? min(tt0 + kTile * (G / 2), last_row) : tt0;
            r.kp = *reinterpret_cast<const u32x4*>(kpsrc + (int64_t)(gt / GS) * D);
        }
    };
    // stage a tile in this wave's LDS (the even tile of a pair also stages the side data: V
    // (scale, zero) as fp32 pairs, K group rows); returns whether this lane holds a V scale at or
    // above the current bound 2^e_s
    auto stage_codes = [&](const CodeRegs& r, int par) {
        uint8_t* skt = sk + par * (kTile * D / 2);
        uint8_t* svt = sv + par * (kTile * D / 2);
        *reinterpret_cast<u32x4*>(skt + 16 * lane) = r.k[0];
        *reinterpret_cast<u32x4*>(skt + 16 * lane + 1024) = r.k[1];
        *reinterpret_cast<u32x4*>(svt + 16 * lane) = r.v[0];
        *reinterpret_cast<u32x4*>(svt + 16 * lane + 1024) = r.v[1];
    };
    auto stage_side = [&](const SideRegs& r, bool new_grp) -> bool {
        float smax;
        if constexpr (NG == 1) {
            smax = bf_lo(r.vs[0]);
            reinterpret_cast<float2*>(ssz)[lane] = make_float2(smax, bf_lo(r.vz[0]));
        } else {
#pragma unroll
            for (int w = 0; w < SW; ++w) {
                const float s0 = bf_lo(r.vs[w]), s1 = bf_hi(r.vs[w]);
                reinterpret_cast<float4*>(ssz)[lane * SW + w] = make_float4(s0, bf_lo(r.vz[w]), s1, bf_hi(r.vz[w]));
                smax = w == 0 ? vmax2(s0, s1) : vmax3(smax, s0, s1);
            }
        }
        if constexpr (!ROT) {
            // fp16(64 + z_V) of token lane % 32 of tile lane / 32, every group (exact: |z| <= 256)
            uint16_t* zt = sm.lp.zf[wv] + (lane / kTile) * (NG * kTile) + lane % kTile;
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) {
                const uint32_t zw = r.vz[gI / 2];
                const float z = (gI % 2) ? bf_hi(zw) : bf_lo(zw);
                zt[gI * kTile] = __builtin_bit_cast(uint16_t, (_Float16)(64.0f + z));
            }
        }
        if constexpr (ROT) {
            float* kst = sm.lp.ksz[wv];
            if constexpr (NG == 1) {
                reinterpret_cast<float2*>(kst)[lane] = make_float2(bf_lo(r.ks[0]), bf_lo(r.kz[0]));
            } else {
#pragma unroll
                for (int w = 0; w < SW; ++w)
                    reinterpret_cast<float4*>(kst)[lane * SW + w] =
                        make_float4(bf_lo(r.ks[w]), bf_lo(r.kz[w]), bf_hi(r.ks[w]), bf_hi(r.kz[w]));
            }
        } else {
            if (GS == 32 || (new_grp && lane < 32)) reinterpret_cast<u32x4*>(skp)[lane] = r.kp;
        }
        return smax >= s_lim;
    };

    // ---- the tiles of a pair from their staged LDS copies (slot par = tile t0 + 32 par) ----
    // K group parameters -> Q'^T operand (fp16 hi + lo) and bias, for the group of tile par
    auto setup_group = [&](int par) {
        const uint16_t* tkp = skp + (GS == 32 ? par * 2 * D : 0);   // this tile's K group rows
        // ---- K group parameters -> Q'^T operand (fp16 hi + lo) and bias ----
            // pass 1: largest |q * s_K| of this lane's chunks (the fp16 range check)
            auto chunk_scaled = [&](int p, float (&qs)[8]) {
                const u32x4 sw = *reinterpret_cast<const u32x4*>(tkp + 32 * G + 8 * chunk_of(p));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qs[2 * e] = qv[p][2 * e] * bf_lo(sw[e]);
                    qs[2 * e + 1] = qv[p][2 * e + 1] * bf_hi(sw[e]);
                }
            };
            float qmax = 0.0f;
#pragma unroll
            for (int p = 0; p < PASS; ++p) {
                float qs[8];
                chunk_scaled(p, qs);
#pragma unroll
                for (int j = 0; j < 8; j += 2) qmax = vmax3_abs(qmax, qs[j], qs[j + 1]);
            }
            lscale = a.qscale;
            int tau = 0;
            const bool big = __any(qmax >= 16384.0f);   // uniform: the scaling below is a scalar branch
            if (big) {
                // out of the fp16 range: scale this query's Q' by 2^-tau, tau from the largest
                // |q * s_K| over its 128 channels (lanes that hold the same query)
                qmax = max_lanes<NQ, (4 * NQ < 16 ? 4 * NQ : 16)>(qmax);
                qmax = max_halves(vmax2(qmax, xor_lane<16>(qmax)));
                tau = __builtin_amdgcn_frexp_expf(qmax) - 14;
                lscale = __builtin_ldexpf(a.qscale, tau);
            }
            // pass 2: per chunk, Q' = q * s_K (* 2^-tau) as fp16 hi + lo, published to LDS for the
            // score MFMAs, and the bias partial sum_c Q'_c (z_c + 64)
            float bz = 0.0f, bsum = 0.0f;
#pragma unroll
            for (int p = 0; p < PASS; ++p) {
                float qs[8];
                chunk_scaled(p, qs);
                if (big) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) qs[j] = __builtin_ldexpf(qs[j], -tau);
                }
                const u32x4 zw = *reinterpret_cast<const u32x4*>(tkp + D + 32 * G + 8 * chunk_of(p));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bz = __builtin_fmaf(qs[2 * e], bf_lo(zw[e]), bz);
                    bz = __builtin_fmaf(qs[2 * e + 1], bf_hi(zw[e]), bz);
                    // the first pair starts the sum (an addition of +0 would cost an instruction)
                    bsum = (p == 0 && e == 0) ? qs[0] + qs[1] : bsum + (qs[2 * e] + qs[2 * e + 1]);
                }
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = qs[kPerm[2 * e]], x1 = qs[kPerm[2 * e + 1]];
                    hw[e] = pack_h2(x0, x1);
                    lw[e] = residual_h2(hw[e], x0, x1);
                }
                *reinterpret_cast<u32x4*>(sqx + lane * PASS * 8 + 8 * p) = u32x4{hw[0], hw[1], hw[2], hw[3]};
                *reinterpret_cast<u32x4*>(sqx + lane * PASS * 8 + 8 * p + 4) = u32x4{lw[0], lw[1], lw[2], lw[3]};
            }
            float bpart = __builtin_fmaf(64.0f, bsum, bz);
            // bias: sum over the distinct chunks of this query, then over the 4 lane groups
            bpart = add_lanes<NQ, (4 * NQ < 16 ? 4 * NQ : 16)>(bpart);
            bpart = add_halves(bpart + xor_lane<16>(bpart));
            c0 = __builtin_fmaf(bpart, lscale, ref);
    };
    // scores of tile par -> lg (lane (n, G): tokens 4G+i (half 0) and 16+4G+i (half 1), i = 0..3;
    // lg = logit - ref)
    auto score_tile = [&](int par, float (&lg)[8]) {
        const uint8_t* skt = sk + par * (kTile * D / 2);
        __builtin_amdgcn_wave_barrier();
        if constexpr (ROT) {
            // chunk kk = channels 32 kk .. 32 kk + 31: lane (n, G) takes dword 4 kk + G of token n's row
            // (staged at byte 16 n + 256 kk + 4 G of the half), one accumulator per K group
            floatx4 scg[2][NG];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int gI = 0; gI < NG; ++gI) scg[hf][gI] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int gI = (32 * kk) / GS;
                const half8 bh = __builtin_bit_cast(half8, rq_hi[kk]), bl = __builtin_bit_cast(half8, rq_lo[kk]);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(skt + 1024 * hf + 16 * n + 256 * kk + 4 * G);
                    const half8 ak = nib8(w);
                    scg[hf][gI] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bh, scg[hf][gI], 0, 0, 0);
                    scg[hf][gI] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bl, scg[hf][gI], 0, 0, 0);
                }
            }
            const float2* tks = reinterpret_cast<const float2*>(sm.lp.ksz[wv] + par * (kTile * NG * 2));
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tl = 16 * hf + 4 * G + i;
                    float acc = 0.0f;
#pragma unroll
                    for (int gI = 0; gI < NG; ++gI) {
                        const float2 sz = tks[tl * NG + gI];
                        acc = __builtin_fmaf(sz.x, __builtin_fmaf(-(64.0f + sz.y), rq_sum[gI], scg[hf][gI][i]), acc);
                    }
                    lg[4 * hf + i] = __builtin_fmaf(acc, rq_scale, -ref);
                }
        } else {
            // chunk kk of Q' for query n % NQ was computed by lane qsrc(kk), pass qpass(kk)
            floatx4 sc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
            const u32x4 kraw0 = *reinterpret_cast<const u32x4*>(skt + 16 * lane);
            const u32x4 kraw1 = *reinterpret_cast<const u32x4*>(skt + 1024 + 16 * lane);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int src = PASS == 4 ? lane : 16 * G + n % NQ + (NQ == 8 ? 8 * (kk % 2) : NQ * kk);
                const int ps = PASS == 4 ? kk : (NQ == 8 ? kk / 2 : 0);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(sqx + src * PASS * 8 + 8 * ps);
                const u32x4 lo = *reinterpret_cast<const u32x4*>(sqx + src * PASS * 8 + 8 * ps + 4);
                const half8 bh = __builtin_bit_cast(half8, hi), bl = __builtin_bit_cast(half8, lo);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const half8 ak = nib8((hf ? kraw1 : kraw0)[kk]);
                    sc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bh, sc[hf], 0, 0, 0);
                    sc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bl, sc[hf], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lg[i] = __builtin_fmaf(sc[0][i], lscale, -c0);
                lg[4 + i] = __builtin_fmaf(sc[1][i], lscale, -c0);
            }
        }
    };
    // the logits themselves (LG), and the masking of tokens past the wave's range
    auto finish_logits = [&](int t0, float (&lg)[8]) {
        const int nvalid = min(kTile, t_hi - t0);
        if constexpr (LG) {
            // the base-2 logits themselves (lg + ref), for the valid tokens of the real queries
            if (n < NQ) {
                float* lrow = a.lgw + (b * a.Hq + h * NQ + n) * a.ldl + t0;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int tb = 16 * hf + 4 * G;
                    const float x0 = lg[4 * hf] + ref, x1 = lg[4 * hf + 1] + ref;
                    const float x2 = lg[4 * hf + 2] + ref, x3 = lg[4 * hf + 3] + ref;
                    if (tb + 3 < nvalid) {
                        *reinterpret_cast<float4*>(lrow + tb) = make_float4(x0, x1, x2, x3);
                    } else {
                        if (tb < nvalid) lrow[tb] = x0;
                        if (tb + 1 < nvalid) lrow[tb + 1] = x1;
                        if (tb + 2 < nvalid) lrow[tb + 2] = x2;
                    }
                }
            }
        }
        if (nvalid < kTile) {   // only the last pair of a range is partial
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * G + i >= nvalid) lg[i] = kNegBig;
                if (16 + 4 * G + i >= nvalid) lg[4 + i] = kNegBig;
            }
        }
    };
    // the softmax reference, once for the ntl tiles of a pair
    auto move_ref = [&](float (&lg)[2][8], int ntl, bool big_s) {
        float lmax = vmax3(vmax3(lg[0][0], lg[0][1], lg[0][2]), vmax3(lg[0][3], lg[0][4], lg[0][5]), vmax2(lg[0][6], lg[0][7]));
        if (ntl > 1)
            lmax = vmax3(lmax, vmax3(vmax3(lg[1][0], lg[1][1], lg[1][2]), vmax3(lg[1][3], lg[1][4], lg[1][5]), lg[1][6]), lg[1][7]);
        if (__any(lmax > thr || big_s)) {
            // move the reference: largest logit of the tiles (+ margin) and largest V scale
            const float tmax = max_halves(vmax2(lmax, xor_lane<16>(lmax)));
            // largest V scale of the tile pair: lane holds token lane's NG scales
            float sm2 = ssz[2 * NG * lane];
#pragma unroll
            for (int gI = 1; gI < NG; ++gI) sm2 = vmax2(sm2, ssz[2 * (NG * lane + gI)]);
            sm2 = max_halves(max_lanes<1, 32>(sm2));
            int e_new = max(e_s, __builtin_amdgcn_frexp_expf(sm2));   // sm2 < 2^frexp_exp
            e_new = min(max(e_new, kEmin), kEmax);
            const float d = vmax2(thr, tmax + kMargin) + (float)(e_new - 15);
            const float alpha = started ? __builtin_amdgcn_exp2f(-d) : 0.0f;
            l_part *= alpha;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) acc_o[nb] *= alpha;
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) {
                acc_off[gI] *= alpha;
                if constexpr (ROT) zsum[gI] *= alpha;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lg[0][i] -= d;
                lg[1][i] -= d;
            }
            ref += d;
            c0 += d;
            e_s = e_new;
            s_lim = __builtin_ldexpf(1.0f, e_s);
            thr = (float)(15 - e_s);
            started = true;
        }
    };
    // probabilities, P' and the value MFMAs of tile par
    auto values_tile = [&](int par, float (&lg)[8]) {
        const float* tsz = ssz + par * (kTile * NG * 2);            // this tile's (scale, zero) pairs
        const uint8_t* svt = sv + par * (kTile * D / 2);
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(lg[i]);
            l_part += p[i];
        }

        // ---- P' = fp16(p * s_V) per V group, and the zero-point term in fp32 ----
        half8 bp[NG];
        {
            // (scale, zero) of token 16*hf + 4G + i, group gI: float2 at (16*hf + 4G + i) * NG + gI
            auto sz2 = [&](int hf, int x) -> float2 {
                return reinterpret_cast<const float2*>(tsz)[(16 * hf + 4 * G) * NG + x];
            };
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // token slots 2e, 2e+1 -> half hf = e / 2, tokens i = 2(e%2), 2(e%2)+1 of that half
                    const int hf = e / 2, i0 = 2 * (e % 2), i1 = i0 + 1;
                    const float2 a0 = sz2(hf, i0 * NG + gI), a1 = sz2(hf, i1 * NG + gI);
                    const float ps0 = p[2 * e] * a0.x, ps1 = p[2 * e + 1] * a1.x;
                    w[e] = pack_h2(ps0, ps1);
                    if constexpr (ROT) {
                        // the output is rotated back afterwards, which gathers an error shared by a
                        // group's channels into a few coordinates: the zero-point term takes the same
                        // fp16 P' the codes are multiplied with, so its rounding cancels inside
                        // (code - z); below the fp16 normal range (tiny scales of constant groups) P'
                        // has lost its precision and the unrounded p * s_V is used instead
                        const half2v hw2 = __builtin_bit_cast(half2v, w[e]);
                        const float r0 = (float)hw2[0], r1 = (float)hw2[1];
                        const float u0 = r0 >= 6.103515625e-05f ? r0 : ps0, u1 = r1 >= 6.103515625e-05f ? r1 : ps1;
                        zsum[gI] = __builtin_fmaf(u0, a0.y, zsum[gI]);
                        zsum[gI] = __builtin_fmaf(u1, a1.y, zsum[gI]);
                    }
                }
                bp[gI] = as_half8(w[0], w[1], w[2], w[3]);
            }
        }

        // ---- values: V codes^T from the LDS tile, 8 + NG MFMAs ----
        {
            const int tok[8] = {4 * G, 4 * G + 1, 4 * G + 2, 4 * G + 3,
                                16 + 4 * G, 16 + 4 * G + 1, 16 + 4 * G + 2, 16 + 4 * G + 3};
            const half8 c64 = as_half8(kMagic, kMagic, kMagic, kMagic);
            const uint16_t* tzf = sm.lp.zf[wv] + par * (NG * kTile);
#pragma unroll
            for (int gI = 0; gI < NG; ++gI) {
                // this lane's piece of group gI: PB bytes at byte offset (GS/2)*gI + PB*n
                const int boff = (GS / 2) * gI + PB * n;
                // dword per token pair: the pair's pieces side by side (token a low, token b high)
                uint32_t P[4][2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint8_t* ra = svt + tok[2 * e] * (D / 2) + boff;
                    const uint8_t* rb = svt + tok[2 * e + 1] * (D / 2) + boff;
                    if constexpr (PB == 1) {
                        P[e][0] = (uint32_t)*ra | ((uint32_t)*rb << 16);                        // [a 0 b 0]
                    } else if constexpr (PB == 2) {
                        P[e][0] = (uint32_t)*reinterpret_cast<const uint16_t*>(ra) |
                                  ((uint32_t)*reinterpret_cast<const uint16_t*>(rb) << 16);     // [a0 a1 b0 b1]
                    } else {
                        const uint32_t wa = *reinterpret_cast<const uint32_t*>(ra);
                        const uint32_t wb = *reinterpret_cast<const uint32_t*>(rb);
                        P[e][0] = __builtin_amdgcn_perm(wb, wa, 0x05040100u);                  // [a0 a1 b0 b1]
                        P[e][1] = __builtin_amdgcn_perm(wb, wa, 0x07060302u);                  // [a2 a3 b2 b3]
                    }
                }
                // nibble k of both tokens -> fp16(64 + code) pair: move it to bits 4..7 / 20..23
#pragma unroll
                for (int k = 0; k < BPG; ++k) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t src = P[e][k / 4];
                        const int kb = k % 4;   // byte kb / 2 of each token, low nibble when kb is even
                        const uint32_t x = kb == 0 ? (src << 4) : kb == 1 ? src : kb == 2 ? (src >> 4) : (src >> 8);
                        w[e] = nib_pair(x);
                    }
                    const int nb = gI * BPG + k;
                    acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(w[0], w[1], w[2], w[3]), bp[gI],
                                                                       acc_o[nb], 0, 0, 0);
                }
                if constexpr (ROT) {
                    acc_off[gI] = __builtin_amdgcn_mfma_f32_16x16x32_f16(c64, bp[gI], acc_off[gI], 0, 0, 0);
                } else {
                    // sum_t P'[t][n] * (64 + z_V[t][gI]) in one MFMA: every row of A is the token slots'
                    // fp16(64 + z), in the order of bp's slots (tokens 4G..4G+3, then 16+4G..16+4G+3)
                    const uint2 z0 = *reinterpret_cast<const uint2*>(tzf + gI * kTile + 4 * G);
                    const uint2 z1 = *reinterpret_cast<const uint2*>(tzf + gI * kTile + 16 + 4 * G);
                    acc_off[gI] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(z0.x, z0.y, z1.x, z1.y), bp[gI],
                                                                         acc_off[gI], 0, 0, 0);
                }
            }
        }
    };

    // Tile i of the wave starts at t_lo + 32 i.  Each step stages a pair of tiles, refills their
    // registers a pair ahead and computes the pair: both tiles' scores (their MFMA chains are
    // independent), one update of the softmax reference for the 64 tokens, then each tile's values.
    // A tile at or past t_hi (the odd one of the last pair, at most) is fully masked.  Loads past the
    // wave's last tile re-read that tile, which is still in cache.
    if (t_lo < t_hi) {
        const int ntile = (t_hi - t_lo + kTile - 1) / kTile;
        const int t_last = t_lo + (ntile - 1) * kTile;
        auto tile_at = [&](int i) { return min(t_lo + i * kTile, t_last); };
        CodeRegs ce, co;
        SideRegs sd;
        // issue order: even tile, its side data, odd tile (the schedule must keep it: the first
        // wait counts on it)
        fetch_codes(ce, tile_at(0));
        fetch_side(sd, tile_at(0));
        __builtin_amdgcn_sched_barrier(0);
        fetch_codes(co, tile_at(1));
        __builtin_amdgcn_sched_barrier(0);
        for (int i = 0; i < ntile; i += 2) {
            const int tt = t_lo + i * kTile;
            const bool new_grp = (tt % GS == 0) || (i == 0);
            stage_codes(ce, 0);
            const bool big_s = stage_side(sd, new_grp);
            fetch_codes(ce, tile_at(i + 2));
            fetch_side(sd, tile_at(i + 2));
            __builtin_amdgcn_sched_barrier(0);
            stage_codes(co, 1);
            fetch_codes(co, tile_at(i + 3));
            __builtin_amdgcn_wave_barrier();
            float lg[2][8];
            if (!ROT && new_grp) setup_group(0);
            score_tile(0, lg[0]);
            if (!ROT && GS == 32) setup_group(1);   // the odd tile starts the next group of 32
            score_tile(1, lg[1]);
            finish_logits(tt, lg[0]);
            finish_logits(tt + kTile, lg[1]);
            move_ref(lg, 2, big_s);
            values_tile(0, lg[0]);
            values_tile(1, lg[1]);
            __builtin_amdgcn_wave_barrier();     // LDS reads done before the next pair overwrites
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---------------- finish the wave: sums over the 4 lane groups, offset and zero terms ----------------
    l_part = add_halves(l_part + xor_lane<16>(l_part));
    if constexpr (ROT) {
#pragma unroll
        for (int gI = 0; gI < NG; ++gI) {
            zsum[gI] = add_halves(zsum[gI] + xor_lane<16>(zsum[gI]));
        }
    }
    __syncthreads();   // every wave is done with the loop buffers before the merge reuses them
    // acc_o[nb][i] is channel row m = 4G + i of block nb, query n
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int gI = nb / BPG, k = nb % BPG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * G + i;
            const int c = GS * gI + BPG * m + k;
            sm.mg.o[wv][n][c] = acc_o[nb][i] - acc_off[gI][i] - zsum[gI];
        }
    }
    if (G == 0) {
        sm.mg.m[wv][n] = started ? ref : kNegBig;
        sm.mg.l[wv][n] = l_part;
    }
    __syncthreads();
    // merge the 4 waves and write (m, l, acc[D]) for each real query
    for (int e = tid; e < NQ * D; e += kThreads) {
        const int qn = e / D, c = e % D;
        float M = sm.mg.m[0][qn];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = vmax2(M, sm.mg.m[w][qn]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2f(sm.mg.m[w][qn] - M);
            L = __builtin_fmaf(sm.mg.l[w][qn], f, L);
            A = __builtin_fmaf(sm.mg.o[w][qn][c], f, A);
        }
        float* dst = a.ws + ((b * a.Hq + h * NQ + qn) * a.nslot + split) * (D + 2);
        if (c == 0) { dst[0] = M; dst[1] = L; }
        dst[2 + c] = A;
    }
}

template <int GS, bool LG>
void launch_nq(const MfmaArgs& a, int nq, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H * (a.nsplit + a.nres))), blk(kThreads);
    switch (nq) {
        case 1: hipLaunchKernelGGL((attn_mfma_kernel<GS, 1, LG>), grid, blk, 0, st, a); break;
        case 2: hipLaunchKernelGGL((attn_mfma_kernel<GS, 2, LG>), grid, blk, 0, st, a); break;
        case 4: hipLaunchKernelGGL((attn_mfma_kernel<GS, 4, LG>), grid, blk, 0, st, a); break;
        case 8: hipLaunchKernelGGL((attn_mfma_kernel<GS, 8, LG>), grid, blk, 0, st, a); break;
        default: hipLaunchKernelGGL((attn_mfma_kernel<GS, 16, LG>), grid, blk, 0, st, a); break;
    }
}

template <int GS>
void launch_nq_rot(const MfmaArgs& a, int nq, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H * a.nsplit)), blk(kThreads);
    switch (nq) {
        case 1: hipLaunchKernelGGL((attn_mfma_kernel<GS, 1, false, true>), grid, blk, 0, st, a); break;
        case 2: hipLaunchKernelGGL((attn_mfma_kernel<GS, 2, false, true>), grid, blk, 0, st, a); break;
        case 4: hipLaunchKernelGGL((attn_mfma_kernel<GS, 4, false, true>), grid, blk, 0, st, a); break;
        case 8: hipLaunchKernelGGL((attn_mfma_kernel<GS, 8, false, true>), grid, blk, 0, st, a); break;
        default: hipLaunchKernelGGL((attn_mfma_kernel<GS, 16, false, true>), grid, blk, 0, st, a); break;
    }
}

template <bool LG>
void launch_g(const MfmaArgs& a, int64_t g, int nq, hipStream_t st) {
    if (g == 32) launch_nq<32, LG>(a, nq, st);
    else if (g == 64) launch_nq<64, LG>(a, nq, st);
    else launch_nq<128, LG>(a, nq, st);
}

}  // namespace

int res_splits(int64_t R) { return (int)cdiv(R, kResTile); }

// attn_waves of the instance launch_attn_mfma picks for these arguments (lg: logits written)
int mfma_waves(int64_t g, int64_t nq, bool lg) {
    return (!lg && g >= 64 && nq <= 4) ? 3 : 2;
}

// Launch the INT4 token range [0, Tq) on the matrix cores (d = 128) and the bf16 residual
// [Tq, T) in blocks of the same grid.  Partials go to ws slots 0 .. nsplit-1 (INT4) and
// nsplit .. nsplit + res_splits(R) - 1 (residual) of each (b, hq); nslot is their sum.  With lgw,
// every token's base-2 logit also goes to lgw[(b * Hq + hq) * ldl + t].
void launch_attn_mfma(const kvq_int4_cache* c, const void* q, int64_t Hq, float qscale, float* ws, int nsplit,
                      int64_t split_len, int nslot, float* lgw, int64_t ldl, hipStream_t st) {
    MfmaArgs a;
    a.k_codes = c->k_codes; a.k_scale = c->k_scale; a.k_zero = c->k_zero;
    a.v_codes = c->v_codes; a.v_scale = c->v_scale; a.v_zero = c->v_zero;
    a.k_res = c->k_res; a.v_res = c->v_res;
    a.R = (int)c->R;
    a.nres = res_splits(c->R);
    a.q = static_cast<const uint16_t*>(q);
    a.ws = ws;
    a.lgw = lgw;
    a.ldl = ldl;
    a.B = c->B; a.H = c->H; a.Hq = Hq;
    a.Tq = (int)(c->T - c->R); a.nKg = (int)cdiv(a.Tq, c->g);
    a.ldq = c->cap ? c->cap : a.Tq;
    a.ldk = cdiv(a.ldq, c->g);
    a.ldr = c->rcap ? c->rcap : c->R;
    a.split_len = (int)split_len;
    a.nsplit = nsplit;
    a.nslot = nslot;
    a.qscale = qscale;
    const int nq = (int)(Hq / c->H);
    if (lgw) launch_g<true>(a, c->g, nq, st);
    else launch_g<false>(a, c->g, nq, st);
}

// The rotated per-token cache (d = 128): all T tokens on the matrix cores, no bf16 window.
// qrot: rotated queries [B][Hq][128] fp32 (times sm_scale * log2 e); partials to ws slots
// 0 .. nsplit - 1 of each (b, hq) in the layout the rotated combine reads.
void launch_attn_mfma_rot(const kvq_rot_cache* c, const float* qrot, int64_t Hq, float* ws, int nsplit,
                          int64_t split_len, hipStream_t st) {
    MfmaArgs a{};
    a.k_codes = c->k_codes; a.k_scale = c->k_scale; a.k_zero = c->k_zero;
    a.v_codes = c->v_codes; a.v_scale = c->v_scale; a.v_zero = c->v_zero;
    a.k_res = nullptr; a.v_res = nullptr;
    a.R = 0;
    a.nres = 0;
    a.q = nullptr;
    a.qrot = qrot;
    a.ws = ws;
    a.lgw = nullptr;
    a.ldl = 0;
    a.B = c->B; a.H = c->H; a.Hq = Hq;
    a.Tq = (int)c->T; a.nKg = 0;
    a.ldq = c->T;
    a.ldk = 0;
    a.ldr = 0;
    a.split_len = (int)split_len;
    a.nsplit = nsplit;
    a.nslot = nsplit;
    a.qscale = 1.0f;
    const int nq = (int)(Hq / c->H);
    if (c->g == 32) launch_nq_rot<32>(a, nq, st);
    else if (c->g == 64) launch_nq_rot<64>(a, nq, st);
    else launch_nq_rot<128>(a, nq, st);
}

}  // namespace kvq
