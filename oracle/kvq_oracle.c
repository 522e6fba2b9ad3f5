/* kvq_oracle.c -- TEST INFRASTRUCTURE ONLY (see kvq_oracle.h).
 *
 * A plain, slow, obviously-correct CPU reference.  Sources, cited by page
 * title and section:
 *   [Walkthrough]  "KV Compression 公式到源码对照" (formula-to-code walkthrough),
 *                  sections 1.1, 1.2, 1.3, 2, 3.1, 3.2, 3.3, 4.
 *   [Explainer]    "KV cache 压缩：把历史装得更小" (animated KV-cache compression
 *                  explainer), sections on quantization, the worked 4-bit
 *                  example, the group-size table, the residual budget, the
 *                  grouping axis, K/V error propagation and byte accounting.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off (no FMA contraction, no fast-math;
 * the default x86-64 target has no FMA and rounds to nearest-even).
 *
 * Readings where the pages leave a step open are marked READING and listed
 * in the design notes.
 */
#include "kvq_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* fp32(1e-8): the floor the walkthrough clips the absmax / range to (§1.1, §1.2). */
static const float RANGE_FLOOR = 1e-8f;

/* ---------------------------------------------------------------- bf16 ---- */

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round an fp32 value to the nearest bf16, ties to an even bf16 significand. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays NaN */
    uint32_t kept = u & 0xffff0000u;   /* the bf16 next to f, toward zero */
    uint32_t dropped = u & 0x0000ffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 0x00010000u)))
        kept += 0x00010000u;            /* one bf16 step away from zero */
    return (uint16_t)(kept >> 16);
}

/* Smallest bf16 >= f, for finite f > 0 (READING: scales are stored rounded up so
 * that every value of a group stays within half a step of a level). */
static uint16_t bf16_round_up_positive(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t kept = u & 0xffff0000u;
    if (u & 0x0000ffffu) kept += 0x00010000u;
    return (uint16_t)(kept >> 16);
}

void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

static float load_elem(const void* x, int is_bf16, int64_t i) {
    if (is_bf16) return orc_bf16_to_f32(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

/* Integer value of round-half-even, kept in double so nothing overflows. */
static double clampd(double v, double lo, double hi) {
    if (v < lo) return lo;
    if (v > hi) return hi;
    return v;
}

/* -------------------------------------------------- per-channel, §1.1-1.3 -- */

/* [Walkthrough §1.1] scale_c = max|x_c| / qmax (absmax clipped below at 1e-8),
 * q = clip(round(x / scale_c), -qmax, qmax), qmax = 2^(bits-1) - 1.
 * Channels are the columns of each [R][C] slice; the max runs over the rows. */
int orc_quant_sym(const void* x, int x_bf16, int64_t nb, int64_t R, int64_t C, int bits,
                  int8_t* q, float* scale, int8_t* zp) {
    if (nb <= 0 || R <= 0 || C <= 0 || bits < 2 || bits > 8) return -1;
    const int qmax = (1 << (bits - 1)) - 1;
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t base = b * R * C;
        for (int64_t c = 0; c < C; ++c) {
            float absmax = 0.0f;
            for (int64_t r = 0; r < R; ++r) {
                float a = fabsf(load_elem(x, x_bf16, base + r * C + c));
                if (a > absmax) absmax = a;
            }
            if (absmax < RANGE_FLOOR) absmax = RANGE_FLOOR;
            const float s = absmax / (float)qmax;
            scale[b * C + c] = s;
            if (zp) zp[b * C + c] = 0;
            for (int64_t r = 0; r < R; ++r) {
                const float v = load_elem(x, x_bf16, base + r * C + c);
                const float n = rintf(v / s); /* np.round: half to even */
                q[base + r * C + c] = (int8_t)clampd((double)n, -qmax, qmax);
            }
        }
    }
    return 0;
}

/* [Walkthrough §1.2] scale = (max - min) / (qmax - qmin) (range clipped below at 1e-8),
 * zero_point = round(qmin - min / scale) as int8, q = clip(round(x / scale) + zero_point,
 * qmin, qmax).  The zero point is added after rounding, as in the page's code.
 * READING: a zero point outside the int8 range saturates. */
int orc_quant_asym(const void* x, int x_bf16, int64_t nb, int64_t R, int64_t C, int qmin, int qmax,
                   int8_t* q, float* scale, int8_t* zp) {
    if (nb <= 0 || R <= 0 || C <= 0 || qmin >= qmax || qmin < -128 || qmax > 127) return -1;
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t base = b * R * C;
        for (int64_t c = 0; c < C; ++c) {
            float mn = load_elem(x, x_bf16, base + c), mx = mn;
            for (int64_t r = 1; r < R; ++r) {
                const float v = load_elem(x, x_bf16, base + r * C + c);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            float range = mx - mn;
            if (range < RANGE_FLOOR) range = RANGE_FLOOR;
            const float s = range / (float)(qmax - qmin);
            const float zr = rintf((float)qmin - mn / s);
            const int z = (int)clampd((double)zr, -128.0, 127.0);
            scale[b * C + c] = s;
            zp[b * C + c] = (int8_t)z;
            for (int64_t r = 0; r < R; ++r) {
                const float v = load_elem(x, x_bf16, base + r * C + c);
                const double code = (double)rintf(v / s) + (double)z;
                q[base + r * C + c] = (int8_t)clampd(code, qmin, qmax);
            }
        }
    }
    return 0;
}

/* [Walkthrough §1.3] x_hat = (q - zero_point) * scale; the difference is formed in fp32
 * (exact for int8 operands) and multiplied once. */
void orc_dequant_pc(const int8_t* q, const float* scale, const int8_t* zp,
                    int64_t nb, int64_t R, int64_t C, float* out) {
    for (int64_t b = 0; b < nb; ++b)
        for (int64_t r = 0; r < R; ++r)
            for (int64_t c = 0; c < C; ++c) {
                const int64_t i = (b * R + r) * C + c;
                const float z = zp ? (float)zp[b * C + c] : 0.0f;
                out[i] = ((float)q[i] - z) * scale[b * C + c];
            }
}

/* [Walkthrough §1.3] RMSE = sqrt(sum (x - x_hat)^2 / N), max and mean absolute error.
 * READING: accumulated in fp64 in flat index order. */
void orc_err_stats(const void* x, int x_bf16, const void* xh, int xh_bf16, int64_t n, double out[3]) {
    double sq = 0.0, ab = 0.0, mx = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double e = (double)load_elem(x, x_bf16, i) - (double)load_elem(xh, xh_bf16, i);
        sq += e * e;
        ab += fabs(e);
        if (fabs(e) > mx) mx = fabs(e);
    }
    out[0] = sq;
    out[1] = ab;
    out[2] = mx;
}

void orc_stats_finalize(const double in[3], int64_t n, double* rmse, double* max_abs, double* mean_abs) {
    *rmse = sqrt(in[0] / (double)n);
    *max_abs = in[2];
    *mean_abs = in[1] / (double)n;
}

/* ------------------------------------------------ 4-bit groups (Explainer) -- */

/* One affine 4-bit group.  [Explainer, quantization section] x ~ s * (q - z) with a
 * bf16 scale and a bf16 zero stored per group; the integer steps are those of
 * [Walkthrough §1.2] with qmin = 0, qmax = 15:
 *   s = (max - min) / 15 (range clipped at 1e-8), raised to |min| / 256 when that is
 *       larger, stored as bf16 rounded up (READING: bf16 holds every integer of
 *       magnitude <= 256 exactly, so with s >= |min| / 256 the zero point below is
 *       stored exactly and the 16 levels (k - z) * s cover [min, max]; this keeps the
 *       lab section's round-trip bound |x - x_hat| <= s / 2 for every group; a group
 *       that straddles zero always has range >= |min|, so its scale is unchanged),
 *   z = round(0 - min / s) with the stored s, stored as bf16 (exact: |z| <= 256),
 *   q = clip(round(x / s) + z, 0, 15) with the stored s and z. */
static void int4_group(const float* v, int64_t n, uint16_t* s_out, uint16_t* z_out, uint8_t* codes) {
    float mn = v[0], mx = v[0];
    for (int64_t i = 1; i < n; ++i) {
        if (v[i] < mn) mn = v[i];
        if (v[i] > mx) mx = v[i];
    }
    float range = mx - mn;
    if (range < RANGE_FLOOR) range = RANGE_FLOOR;
    float s32 = range / 15.0f;
    const float zfloor = fabsf(mn) / 256.0f;
    if (zfloor > s32) s32 = zfloor;
    const uint16_t sb = bf16_round_up_positive(s32);
    const float s = orc_bf16_to_f32(sb);
    const float zr = rintf(0.0f - mn / s);
    const uint16_t zb = orc_f32_to_bf16(zr);
    const float z = orc_bf16_to_f32(zb);
    for (int64_t i = 0; i < n; ++i) {
        const double code = (double)rintf(v[i] / s) + (double)z;
        codes[i] = (uint8_t)clampd(code, 0.0, 15.0);
    }
    *s_out = sb;
    *z_out = zb;
}

/* Nibble packing: byte j of a row holds the code of channel 2j in its low nibble and
 * channel 2j+1 in its high nibble (READING: the pages fix 4 bits per number only). */
static void pack_row(const uint8_t* codes, int64_t d, uint8_t* out) {
    for (int64_t j = 0; j < d / 2; ++j) out[j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* [Explainer, grouping-axis and residual-budget sections] K is grouped per channel across
 * g consecutive tokens (the last group of a channel may be partial), V per token across g
 * consecutive channels; the last R tokens stay bf16.  Output layouts:
 *   codes  u8   [B][H][Tq][d/2]        (Tq = T - R)
 *   K s/z  bf16 [B][H][ceil(Tq/g)][d]
 *   V s/z  bf16 [B][H][Tq][d/g]
 *   res    bf16 [B][H][R][d]                                                  */
int orc_int4_quant(const uint16_t* K, const uint16_t* V, int64_t B, int64_t T, int64_t H, int64_t d,
                   int64_t g, int64_t R,
                   uint8_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                   uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                   uint16_t* k_res, uint16_t* v_res) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || d % 2 || g <= 0 || d % g || R < 0 || R > T) return -1;
    const int64_t Tq = T - R, nKg = ceil_div(Tq, g);
    float* vals = (float*)malloc(sizeof(float) * (size_t)(g > d ? g : d));
    uint8_t* cg = (uint8_t*)malloc((size_t)(g > d ? g : d));
    uint8_t* row = (uint8_t*)malloc((size_t)d);
    uint8_t* kq = (uint8_t*)malloc((size_t)(Tq > 0 ? Tq : 1) * (size_t)d); /* unpacked K codes of one (b,h) */
    if (!vals || !cg || !row || !kq) { free(vals); free(cg); free(row); free(kq); return -2; }

    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            /* K: per channel c, per token group j */
            for (int64_t j = 0; j < nKg; ++j) {
                const int64_t t0 = j * g, n = (t0 + g <= Tq) ? g : Tq - t0;
                for (int64_t c = 0; c < d; ++c) {
                    for (int64_t i = 0; i < n; ++i)
                        vals[i] = orc_bf16_to_f32(K[((b * T + t0 + i) * H + h) * d + c]);
                    const int64_t mi = ((b * H + h) * nKg + j) * d + c;
                    int4_group(vals, n, &k_scale[mi], &k_zero[mi], cg);
                    for (int64_t i = 0; i < n; ++i) kq[(t0 + i) * d + c] = cg[i];
                }
            }
            for (int64_t t = 0; t < Tq; ++t) pack_row(&kq[t * d], d, &k_codes[((b * H + h) * Tq + t) * (d / 2)]);

            /* V: per token t, per channel group k */
            for (int64_t t = 0; t < Tq; ++t) {
                for (int64_t k = 0; k < d / g; ++k) {
                    for (int64_t i = 0; i < g; ++i)
                        vals[i] = orc_bf16_to_f32(V[((b * T + t) * H + h) * d + k * g + i]);
                    const int64_t mi = ((b * H + h) * Tq + t) * (d / g) + k;
                    int4_group(vals, g, &v_scale[mi], &v_zero[mi], &row[k * g]);
                }
                pack_row(row, d, &v_codes[((b * H + h) * Tq + t) * (d / 2)]);
            }

            /* residual: the most recent R tokens, verbatim */
            for (int64_t r = 0; r < R; ++r)
                for (int64_t c = 0; c < d; ++c) {
                    k_res[((b * H + h) * R + r) * d + c] = K[((b * T + Tq + r) * H + h) * d + c];
                    v_res[((b * H + h) * R + r) * d + c] = V[((b * T + Tq + r) * H + h) * d + c];
                }
        }
    free(vals); free(cg); free(row); free(kq);
    return 0;
}

/* x_hat = (q - z) * s, rounded once to fp32 (the fp64 product is exact for |z| < 2^44). */
static float int4_level(unsigned code, uint16_t sb, uint16_t zb) {
    return (float)(((double)code - (double)orc_bf16_to_f32(zb)) * (double)orc_bf16_to_f32(sb));
}

void orc_int4_dequant(int is_k, const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                      const uint16_t* res, int64_t B, int64_t T, int64_t H, int64_t d, int64_t g,
                      int64_t R, float* out) {
    const int64_t Tq = T - R, nKg = ceil_div(Tq, g);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t c = 0; c < d; ++c) {
                    float v;
                    if (t < Tq) {
                        const uint8_t byte = codes[((b * H + h) * Tq + t) * (d / 2) + c / 2];
                        const unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
                        const int64_t mi = is_k ? ((b * H + h) * nKg + t / g) * d + c
                                                : ((b * H + h) * Tq + t) * (d / g) + c / g;
                        v = int4_level(code, scale[mi], zero[mi]);
                    } else {
                        v = orc_bf16_to_f32(res[((b * H + h) * R + (t - Tq)) * d + c]);
                    }
                    out[((b * T + t) * H + h) * d + c] = v;
                }
}

/* ------------------------------------------------------ decode attention --- */

/* Dequantized [T][d] slice of head (b, h) in fp64. */
static void slice_fp64(int is_k, const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                       const uint16_t* res, int64_t b, int64_t h, int64_t T, int64_t H, int64_t d,
                       int64_t g, int64_t R, double* out) {
    const int64_t Tq = T - R, nKg = ceil_div(Tq, g);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < d; ++c) {
            double v;
            if (t < Tq) {
                const uint8_t byte = codes[((b * H + h) * Tq + t) * (d / 2) + c / 2];
                const unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
                const int64_t mi = is_k ? ((b * H + h) * nKg + t / g) * d + c
                                        : ((b * H + h) * Tq + t) * (d / g) + c / g;
                v = (double)int4_level(code, scale[mi], zero[mi]);
            } else {
                v = (double)orc_bf16_to_f32(res[((b * H + h) * R + (t - Tq)) * d + c]);
            }
            out[t * d + c] = v;
        }
}

/* softmax(sm_scale * q . k_t) . v over all T tokens, fp64 ([Explainer] the attention kernel
 * reads the low-bit cache and dequantizes it; GQA: query head hq reads KV head
 * hq / (Hq / Hkv), consecutive query heads sharing one KV head). */
static void attend_row(const double* kh, const double* vh, int64_t T, int64_t d,
                       const uint16_t* qrow, double sm_scale, double* logit, double* o, double* probs) {
    double m = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += (double)orc_bf16_to_f32(qrow[c]) * kh[t * d + c];
        logit[t] = sm_scale * acc;
        if (logit[t] > m) m = logit[t];
    }
    double Z = 0.0;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const double p = exp(logit[t] - m);
        Z += p;
        for (int64_t c = 0; c < d; ++c) o[c] += p * vh[t * d + c];
    }
    for (int64_t c = 0; c < d; ++c) o[c] /= Z;
    /* the attention weights themselves, softmax(sm_scale * q . k_t) over t */
    if (probs)
        for (int64_t t = 0; t < T; ++t) probs[t] = exp(logit[t] - m) / Z;
}

int orc_decode_attn_rows(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                         const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                         const uint16_t* k_res, const uint16_t* v_res,
                         int64_t B, int64_t T, int64_t Hkv, int64_t d, int64_t g, int64_t R,
                         const uint16_t* q, int64_t Hq, double sm_scale,
                         const int64_t* rows_b, const int64_t* rows_hq, int64_t n_rows, double* out,
                         double* probs) {
    if (B <= 0 || T <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || d <= 0 || d % g || R < 0 || R > T) return -1;
    double* kh = (double*)malloc(sizeof(double) * (size_t)(T * d));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(T * d));
    double* lg = (double*)malloc(sizeof(double) * (size_t)T);
    if (!kh || !vh || !lg) { free(kh); free(vh); free(lg); return -2; }
    int64_t cur_b = -1, cur_h = -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t b = rows_b[i], hq = rows_hq[i], h = hq / (Hq / Hkv);
        if (b != cur_b || h != cur_h) {
            slice_fp64(1, k_codes, k_scale, k_zero, k_res, b, h, T, Hkv, d, g, R, kh);
            slice_fp64(0, v_codes, v_scale, v_zero, v_res, b, h, T, Hkv, d, g, R, vh);
            cur_b = b;
            cur_h = h;
        }
        attend_row(kh, vh, T, d, &q[(b * Hq + hq) * d], sm_scale, lg, &out[i * d], probs ? &probs[i * T] : NULL);
    }
    free(kh); free(vh); free(lg);
    return 0;
}

int orc_decode_attn(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                    const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                    const uint16_t* k_res, const uint16_t* v_res,
                    int64_t B, int64_t T, int64_t Hkv, int64_t d, int64_t g, int64_t R,
                    const uint16_t* q, int64_t Hq, double sm_scale, double* out) {
    if (B <= 0 || Hq <= 0) return -1;
    int64_t* rb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B * Hq));
    int64_t* rh = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B * Hq));
    if (!rb || !rh) { free(rb); free(rh); return -2; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t hq = 0; hq < Hq; ++hq) {
            rb[b * Hq + hq] = b;
            rh[b * Hq + hq] = hq;
        }
    const int rc = orc_decode_attn_rows(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, k_res, v_res,
                                        B, T, Hkv, d, g, R, q, Hq, sm_scale, rb, rh, B * Hq, out, NULL);
    free(rb); free(rh);
    return rc;
}

/* ------------------------------------------------------ token selection ---- */

/* [Walkthrough §3.1] Score(i) = sum over observed steps of a_t(i), an fp32 sum over
 * axis 0 of the [num_steps][num_tokens] history.  READING: sequential in t from 0. */
void orc_colsum(const float* hist, int64_t rows, int64_t T_obs, int64_t T, float* scores) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* hr = hist + r * T_obs * T;
        float* sr = scores + r * T;
        for (int64_t j = 0; j < T; ++j) sr[j] = 0.0f;
        for (int64_t t = 0; t < T_obs; ++t)
            for (int64_t j = 0; j < T; ++j) sr[j] = sr[j] + hr[t * T + j];
    }
}

/* Number of indices keep_recent_and_heavy_hitters returns: the union of the recent
 * window and TopK over the rest, min(T, max(budget, min(window, T))). */
int64_t orc_keep_count(int64_t T, int64_t budget, int64_t window) {
    const int64_t recent = window < T ? window : T;
    const int64_t k = budget > recent ? budget : recent;
    return k < T ? k : T;
}

/* Ranking used by TopK: larger score first; equal scores -> lower index first;
 * NaN below every number (READING: the page does not show its TopK helper).  The
 * recent tokens, whose scores were replaced by -inf, rank below every earlier token,
 * NaN included (READING: for numeric scores this is what the -inf mask does; it also
 * keeps |recent ∪ TopK| = min(T, max(budget, |recent|)) when earlier scores are NaN). */
/* qsort has no context argument: the ranking context is per thread, so independent rows may be
 * selected on several threads at once */
static _Thread_local const float* g_rank_vals;
static _Thread_local int64_t g_rank_rs;        /* first recent index */
static int rank_cmp(const void* pa, const void* pb) {
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    const int ra = a >= g_rank_rs, rb = b >= g_rank_rs;
    if (ra != rb) return ra ? 1 : -1;
    const float va = g_rank_vals[a], vb = g_rank_vals[b];
    const int na = isnan(va), nbn = isnan(vb);
    if (na != nbn) return na ? 1 : -1;
    if (!na && va != vb) return va > vb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* [Walkthrough §3.2, §3.3] recent = [max(0, T - W), T); the scores of the recent
 * tokens are set to -inf; TopK(scores, max(0, B - |recent|)); keep = sorted unique
 * union of recent and the TopK set, as int32. */
static int select_row(const float* scores, int64_t T, int64_t budget, int64_t window, int32_t* keep,
                      float* masked, int32_t* order, unsigned char* flag) {
    const int64_t rs = T - window > 0 ? T - window : 0;
    for (int64_t j = 0; j < T; ++j) masked[j] = j < rs ? scores[j] : -INFINITY;
    int64_t heavy = budget - (T - rs);
    if (heavy < 0) heavy = 0;
    if (heavy > T) heavy = T;
    for (int64_t j = 0; j < T; ++j) order[j] = (int32_t)j;
    g_rank_vals = masked;
    g_rank_rs = rs;
    qsort(order, (size_t)T, sizeof(int32_t), rank_cmp);
    memset(flag, 0, (size_t)T);
    for (int64_t i = 0; i < heavy; ++i) flag[order[i]] = 1;
    for (int64_t j = rs; j < T; ++j) flag[j] = 1;
    int64_t n = 0;
    for (int64_t j = 0; j < T; ++j)
        if (flag[j]) keep[n++] = (int32_t)j;
    return (int)(n == orc_keep_count(T, budget, window) ? 0 : -3);
}

int orc_select(const float* scores, int64_t rows, int64_t T, int64_t budget, int64_t window, int32_t* keep) {
    if (rows <= 0 || T <= 0 || budget < 0 || window < 0 || T > 0x7fffffff) return -1;
    const int64_t K = orc_keep_count(T, budget, window);
    float* masked = (float*)malloc(sizeof(float) * (size_t)T);
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
    unsigned char* flag = (unsigned char*)malloc((size_t)T);
    if (!masked || !order || !flag) { free(masked); free(order); free(flag); return -2; }
    int rc = 0;
    for (int64_t r = 0; r < rows && rc == 0; ++r)
        rc = select_row(scores + r * T, T, budget, window, keep + r * K, masked, order, flag);
    free(masked); free(order); free(flag);
    return rc;
}

int orc_h2o_select(const float* hist, int64_t rows, int64_t T_obs, int64_t T, int64_t budget,
                   int64_t window, float* scores, int32_t* keep) {
    if (rows <= 0 || T_obs <= 0 || T <= 0) return -1;
    orc_colsum(hist, rows, T_obs, T, scores);
    return orc_select(scores, rows, T, budget, window, keep);
}

/* [Explainer, eviction section] eviction keeps only the selected KV: the kept rows of each
 * (b, h) are gathered, in index order, into a dense cache [B][K][H][d]. */
void orc_compact(const uint16_t* src, int64_t B, int64_t T, int64_t H, int64_t d,
                 const int32_t* keep, int64_t K, uint16_t* dst) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t k = 0; k < K; ++k)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t t = keep[(b * H + h) * K + k];
                memcpy(&dst[((b * K + k) * H + h) * d], &src[((b * T + t) * H + h) * d], (size_t)d * 2);
            }
}

/* ------------------------------------------- eviction on the 4-bit cache --- */

/* Current value of token t of head (b, h) in channel c: the dequantized 4-bit level for a
 * quantized token (t < Tq), the stored bf16 value for a residual token. */
static float int4_value(int is_k, const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                        const uint16_t* res, int64_t b, int64_t h, int64_t t, int64_t c,
                        int64_t H, int64_t d, int64_t g, int64_t Tq, int64_t R) {
    if (t >= Tq) return orc_bf16_to_f32(res[((b * H + h) * R + (t - Tq)) * d + c]);
    const int64_t nKg = ceil_div(Tq, g);
    const uint8_t byte = codes[((b * H + h) * Tq + t) * (d / 2) + c / 2];
    const unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
    const int64_t mi = is_k ? ((b * H + h) * nKg + t / g) * d + c : ((b * H + h) * Tq + t) * (d / g) + c / g;
    return int4_level(code, scale[mi], zero[mi]);
}

/* [Explainer, eviction section: only the selected KV is kept; Walkthrough §4: the token
 * saving multiplies the byte saving] applied to a KIVI cache (Explainer, grouping-axis and
 * residual-budget sections).  The K = keep-count kept tokens of every (b, h), in keep
 * order, form a new cache of T2 = K tokens whose last R2 stay bf16.  READING (the pages
 * do not spell out eviction on a grouped 4-bit cache):
 *   - a kept quantized V row keeps its codes, scale and zero (V groups lie inside a token);
 *   - a new K group (g consecutive kept tokens, the last one partial) whose tokens are
 *     exactly all tokens of one old quantized K group, in order, keeps that group's codes,
 *     scale and zero; every other new K group is quantized afresh, per channel, from the
 *     current values of its tokens (the dequantized levels, exact in fp32, or the bf16
 *     residual values) with the steps of int4_group;
 *   - a kept residual token that lands in the quantized part is quantized like a new token
 *     (its V row from its bf16 values, its K channels inside its new group);
 *   - a new residual row holds the current value rounded to the nearest bf16 (the bf16
 *     value itself for a residual token).
 * Output layouts as orc_int4_quant with T2 = K, R2. */
int orc_int4_evict(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                   const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                   const uint16_t* k_res, const uint16_t* v_res,
                   int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, int64_t R,
                   const int32_t* keep, int64_t K, int64_t R2,
                   uint8_t* dk_codes, uint16_t* dk_scale, uint16_t* dk_zero,
                   uint8_t* dv_codes, uint16_t* dv_scale, uint16_t* dv_zero,
                   uint16_t* dk_res, uint16_t* dv_res) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || d % 2 || g <= 0 || d % g || R < 0 || R > T) return -1;
    if (K < 1 || K > T || R2 < 0 || R2 > K) return -1;
    const int64_t Tq = T - R, nKg = ceil_div(Tq, g);
    const int64_t Tq2 = K - R2, nKg2 = ceil_div(Tq2, g);
    float* xk = (float*)malloc(sizeof(float) * (size_t)(K * d));
    float* xv = (float*)malloc(sizeof(float) * (size_t)(K * d));
    float* vals = (float*)malloc(sizeof(float) * (size_t)(g > d ? g : d));
    uint8_t* cg = (uint8_t*)malloc((size_t)(g > d ? g : d));
    uint8_t* row = (uint8_t*)malloc((size_t)d);
    uint8_t* kq = (uint8_t*)malloc((size_t)(Tq2 > 0 ? Tq2 : 1) * (size_t)d);
    if (!xk || !xv || !vals || !cg || !row || !kq) {
        free(xk); free(xv); free(vals); free(cg); free(row); free(kq);
        return -2;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int32_t* kp = &keep[(b * H + h) * K];
            for (int64_t i = 0; i < K; ++i) {
                if (kp[i] < 0 || kp[i] >= T) {
                    free(xk); free(xv); free(vals); free(cg); free(row); free(kq);
                    return -1;
                }
                for (int64_t c = 0; c < d; ++c) {
                    xk[i * d + c] = int4_value(1, k_codes, k_scale, k_zero, k_res, b, h, kp[i], c, H, d, g, Tq, R);
                    xv[i * d + c] = int4_value(0, v_codes, v_scale, v_zero, v_res, b, h, kp[i], c, H, d, g, Tq, R);
                }
            }
            /* K groups of the new quantized part */
            for (int64_t j = 0; j < nKg2; ++j) {
                const int64_t i0 = j * g, n = (i0 + g <= Tq2) ? g : Tq2 - i0;
                const int64_t t0 = kp[i0];
                int whole = t0 < Tq && t0 % g == 0 && n == ((t0 + g <= Tq) ? g : Tq - t0);
                for (int64_t i = 0; whole && i < n; ++i) whole = kp[i0 + i] == t0 + i;
                for (int64_t c = 0; c < d; ++c) {
                    const int64_t mi = ((b * H + h) * nKg2 + j) * d + c;
                    if (whole) {
                        const int64_t si = ((b * H + h) * nKg + t0 / g) * d + c;
                        dk_scale[mi] = k_scale[si];
                        dk_zero[mi] = k_zero[si];
                        for (int64_t i = 0; i < n; ++i) {
                            const uint8_t byte = k_codes[((b * H + h) * Tq + t0 + i) * (d / 2) + c / 2];
                            kq[(i0 + i) * d + c] = (uint8_t)((c & 1) ? (byte >> 4) : (byte & 15u));
                        }
                    } else {
                        for (int64_t i = 0; i < n; ++i) vals[i] = xk[(i0 + i) * d + c];
                        int4_group(vals, n, &dk_scale[mi], &dk_zero[mi], cg);
                        for (int64_t i = 0; i < n; ++i) kq[(i0 + i) * d + c] = cg[i];
                    }
                }
            }
            for (int64_t i = 0; i < Tq2; ++i) pack_row(&kq[i * d], d, &dk_codes[((b * H + h) * Tq2 + i) * (d / 2)]);
            /* V rows of the new quantized part */
            for (int64_t i = 0; i < Tq2; ++i) {
                const int64_t t = kp[i];
                uint8_t* out = &dv_codes[((b * H + h) * Tq2 + i) * (d / 2)];
                for (int64_t k = 0; k < d / g; ++k) {
                    const int64_t mi = ((b * H + h) * Tq2 + i) * (d / g) + k;
                    if (t < Tq) {
                        const int64_t si = ((b * H + h) * Tq + t) * (d / g) + k;
                        dv_scale[mi] = v_scale[si];
                        dv_zero[mi] = v_zero[si];
                        for (int64_t c = k * g; c < k * g + g; ++c) {
                            const uint8_t byte = v_codes[((b * H + h) * Tq + t) * (d / 2) + c / 2];
                            row[c] = (uint8_t)((c & 1) ? (byte >> 4) : (byte & 15u));
                        }
                    } else {
                        for (int64_t c = 0; c < g; ++c) vals[c] = xv[i * d + k * g + c];
                        int4_group(vals, g, &dv_scale[mi], &dv_zero[mi], &row[k * g]);
                    }
                }
                pack_row(row, d, out);
            }
            /* new residual rows */
            for (int64_t r = 0; r < R2; ++r)
                for (int64_t c = 0; c < d; ++c) {
                    dk_res[((b * H + h) * R2 + r) * d + c] = orc_f32_to_bf16(xk[(Tq2 + r) * d + c]);
                    dv_res[((b * H + h) * R2 + r) * d + c] = orc_f32_to_bf16(xv[(Tq2 + r) * d + c]);
                }
        }
    free(xk); free(xv); free(vals); free(cg); free(row); free(kq);
    return 0;
}

/* ------------------------------------------- Hadamard-rotated 4-bit cache --- */

/* [KV-COBRA notes, item 4 (Walsh-Hadamard rotation with fixed random sign flips): an
 * orthogonal Walsh-Hadamard matrix with a fixed random sign flip mixes the coordinates so
 * that every coordinate gets the mean variance before scalar quantization; the vs-QuaRot /
 * TurboQuant remark: rotation removes outliers.]  Calibration-free reading (no low-rank
 * projection): y = (1/sqrt(d)) * H_d * (s (.) x) with H_d the Sylvester Hadamard matrix
 * (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]) and s in {+1, -1}^d given.
 * READING (precision): the transform is evaluated in fp32 as butterflies in a fixed order,
 * stage h = 1, 2, 4, ..., d/2, each pair (j, j + h) with j & h == 0 becoming (a + b, a - b),
 * then one multiply by fp32(1/sqrt(d)); the quantizer's decisions are taken on these values. */
static void fwht_f32(float* y, int64_t d) {
    for (int64_t h = 1; h < d; h *= 2)
        for (int64_t i = 0; i < d; i += 2 * h)
            for (int64_t j = i; j < i + h; ++j) {
                const float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
}

void orc_rotate_f32(const float* x, const int8_t* signs, int64_t n, int64_t d, float* y) {
    const float c = (float)(1.0 / sqrt((double)d));
    for (int64_t r = 0; r < n; ++r) {
        float* yr = &y[r * d];
        for (int64_t k = 0; k < d; ++k) yr[k] = signs[k] < 0 ? -x[r * d + k] : x[r * d + k];
        fwht_f32(yr, d);
        for (int64_t k = 0; k < d; ++k) yr[k] = yr[k] * c;
    }
}

/* The inverse (H_d is symmetric and H_d H_d = d I): x = s (.) ((1/sqrt(d)) * H_d * y), same order. */
void orc_unrotate_f32(const float* y, const int8_t* signs, int64_t n, int64_t d, float* x) {
    const float c = (float)(1.0 / sqrt((double)d));
    for (int64_t r = 0; r < n; ++r) {
        float* xr = &x[r * d];
        for (int64_t k = 0; k < d; ++k) xr[k] = y[r * d + k];
        fwht_f32(xr, d);
        for (int64_t k = 0; k < d; ++k) {
            const float v = xr[k] * c;
            xr[k] = signs[k] < 0 ? -v : v;
        }
    }
}

/* fp64 versions for the attention reference (no rounding to speak of). */
static void rotate_f64(double* y, const int8_t* signs, int64_t d, int inverse) {
    if (!inverse)
        for (int64_t k = 0; k < d; ++k) y[k] = signs[k] < 0 ? -y[k] : y[k];
    for (int64_t h = 1; h < d; h *= 2)
        for (int64_t i = 0; i < d; i += 2 * h)
            for (int64_t j = i; j < i + h; ++j) {
                const double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    const double c = 1.0 / sqrt((double)d);
    for (int64_t k = 0; k < d; ++k) y[k] *= c;
    if (inverse)
        for (int64_t k = 0; k < d; ++k) y[k] = signs[k] < 0 ? -y[k] : y[k];
}

/* Every token of K and V rotated (its own sign vector per side) and quantized per token in
 * groups of g consecutive rotated coordinates with the steps of int4_group (READING: the
 * calibration-free variant keeps a bf16 scale and zero per group instead of the notes'
 * calibrated fixed step; a per-token layout needs no bf16 window).  Layouts:
 *   codes u8 [B][H][T][d/2] (low nibble = even coordinate), scale / zero bf16 [B][H][T][d/g]. */
int orc_rot_quant(const uint16_t* K, const uint16_t* V, int64_t B, int64_t T, int64_t H, int64_t d, int64_t g,
                  const int8_t* k_signs, const int8_t* v_signs,
                  uint8_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                  uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 1 || (d & (d - 1)) || g <= 0 || d % g) return -1;
    float* x = (float*)malloc(sizeof(float) * (size_t)d);
    float* y = (float*)malloc(sizeof(float) * (size_t)d);
    uint8_t* row = (uint8_t*)malloc((size_t)d);
    if (!x || !y || !row) { free(x); free(y); free(row); return -2; }
    for (int side = 0; side < 2; ++side) {
        const uint16_t* X = side ? V : K;
        const int8_t* sg = side ? v_signs : k_signs;
        uint8_t* codes = side ? v_codes : k_codes;
        uint16_t* sc = side ? v_scale : k_scale;
        uint16_t* zr = side ? v_zero : k_zero;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < T; ++t)
                for (int64_t h = 0; h < H; ++h) {
                    for (int64_t c = 0; c < d; ++c) x[c] = orc_bf16_to_f32(X[((b * T + t) * H + h) * d + c]);
                    orc_rotate_f32(x, sg, 1, d, y);
                    const int64_t o = ((b * H + h) * T + t);
                    for (int64_t k = 0; k < d / g; ++k)
                        int4_group(&y[k * g], g, &sc[o * (d / g) + k], &zr[o * (d / g) + k], &row[k * g]);
                    pack_row(row, d, &codes[o * (d / 2)]);
                }
    }
    free(x); free(y); free(row);
    return 0;
}

/* Dequantize one side back to the original coordinates: the levels (q - z) * s (fp32, rounded
 * once), then the inverse rotation in fp32.  out fp32 [B][T][H][d]. */
void orc_rot_dequant(const uint8_t* codes, const uint16_t* scale, const uint16_t* zero, const int8_t* signs,
                     int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, float* out) {
    float* y = (float*)malloc(sizeof(float) * (size_t)d);
    if (!y) return;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t o = ((b * H + h) * T + t);
                for (int64_t c = 0; c < d; ++c) {
                    const uint8_t byte = codes[o * (d / 2) + c / 2];
                    const unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
                    y[c] = int4_level(code, scale[o * (d / g) + c / g], zero[o * (d / g) + c / g]);
                }
                orc_unrotate_f32(y, signs, 1, d, &out[((b * T + t) * H + h) * d]);
            }
    free(y);
}

/* Decode attention over the rotated cache, fp64: q' = R_K q, softmax over t of
 * sm_scale * q' . k'_t with k'_t the rotated levels, o' = sum_t p_t v'_t, out = R_V^-1 o'.
 * Since R_K is orthogonal, q' . k'_t = q . (R_K^-1 k'_t): this is attention over the
 * dequantized, un-rotated cache.  GQA as orc_decode_attn.  out fp64 [B][Hq][d]. */
int orc_rot_decode_attn(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                        const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                        const int8_t* k_signs, const int8_t* v_signs,
                        int64_t B, int64_t T, int64_t Hkv, int64_t d, int64_t g,
                        const uint16_t* q, int64_t Hq, double sm_scale, double* out) {
    if (B <= 0 || T <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || d <= 1 || (d & (d - 1)) || d % g) return -1;
    double* kh = (double*)malloc(sizeof(double) * (size_t)(T * d));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(T * d));
    double* lg = (double*)malloc(sizeof(double) * (size_t)T);
    double* qr = (double*)malloc(sizeof(double) * (size_t)d);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!kh || !vh || !lg || !qr || !o) { free(kh); free(vh); free(lg); free(qr); free(o); return -2; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hkv; ++h) {
            for (int64_t t = 0; t < T; ++t) {
                const int64_t r = (b * Hkv + h) * T + t;
                for (int64_t c = 0; c < d; ++c) {
                    const uint8_t kb = k_codes[r * (d / 2) + c / 2], vb = v_codes[r * (d / 2) + c / 2];
                    kh[t * d + c] = (double)int4_level((c & 1) ? (kb >> 4) : (kb & 15u), k_scale[r * (d / g) + c / g],
                                                       k_zero[r * (d / g) + c / g]);
                    vh[t * d + c] = (double)int4_level((c & 1) ? (vb >> 4) : (vb & 15u), v_scale[r * (d / g) + c / g],
                                                       v_zero[r * (d / g) + c / g]);
                }
            }
            for (int64_t hq = h * (Hq / Hkv); hq < (h + 1) * (Hq / Hkv); ++hq) {
                for (int64_t c = 0; c < d; ++c) qr[c] = (double)orc_bf16_to_f32(q[(b * Hq + hq) * d + c]);
                rotate_f64(qr, k_signs, d, 0);
                double m = -INFINITY;
                for (int64_t t = 0; t < T; ++t) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc += qr[c] * kh[t * d + c];
                    lg[t] = sm_scale * acc;
                    if (lg[t] > m) m = lg[t];
                }
                double Z = 0.0;
                for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    const double p = exp(lg[t] - m);
                    Z += p;
                    for (int64_t c = 0; c < d; ++c) o[c] += p * vh[t * d + c];
                }
                for (int64_t c = 0; c < d; ++c) o[c] /= Z;
                rotate_f64(o, v_signs, d, 1);
                for (int64_t c = 0; c < d; ++c) out[(b * Hq + hq) * d + c] = o[c];
            }
        }
    free(kh); free(vh); free(lg); free(qr); free(o);
    return 0;
}

/* ------------------------------------------- per-token mixed precision --- */

/* [Adaptive-bit blog: §2.1 four precision levels 2/4/8/16 bits, chosen per token by a
 * controller; §3.1 per-token dynamic quantization, symmetric at 2 and 4 bits, asymmetric at 8
 * bits and above; §3.2 a 2-bit precision tag per token (00/01/10/11 = 2/4/8/16 bits) and
 * tokens of one precision stored contiguously.]  The controller is not part of this: the tags
 * are given, packed four to a byte (row r in bits 2(r%4) .. 2(r%4)+1 of byte r/4).
 * READINGS: a row is one token's C channels (the caller decides what a token row spans);
 * 2 and 4 bits use the steps of Walkthrough §1.1 over the row, 8 bits those of §1.2 with
 * qmin = -128, qmax = 127; a 16-bit row keeps its bf16 bits (the page's fp16 is its model's own
 * 16-bit type); the rows of one width go to that width's pool in row order, at
 * slot = number of earlier rows with the same tag; 2-bit codes are 2-bit two's complement, four
 * to a byte (channel 4j+i in bits 2i, 2i+1 of byte j), 4-bit codes 4-bit two's complement, two to
 * a byte (even channel in the low nibble); scales are fp32, the 8-bit zero point int8. */
static int tag_of(const uint8_t* tags, int64_t r) { return (tags[r / 4] >> (2 * (r % 4))) & 3; }

void orc_mixed_plan(const uint8_t* tags, int64_t N, int32_t* slot, int64_t counts[4]) {
    int64_t n[4] = {0, 0, 0, 0};
    for (int64_t r = 0; r < N; ++r) {
        const int t = tag_of(tags, r);
        slot[r] = (int32_t)n[t];
        n[t] += 1;
    }
    for (int k = 0; k < 4; ++k) counts[k] = n[k];
}

int orc_mixed_quant(const uint16_t* x, int64_t N, int64_t C, const uint8_t* tags, const int32_t* slot,
                    uint8_t* q2, float* s2, uint8_t* q4, float* s4, int8_t* q8, float* s8, int8_t* z8,
                    uint16_t* x16) {
    if (N <= 0 || C <= 0 || C % 8) return -1;
    for (int64_t r = 0; r < N; ++r) {
        const int t = tag_of(tags, r);
        const int64_t k = slot[r];
        const uint16_t* row = &x[r * C];
        if (t == 3) {
            memcpy(&x16[k * C], row, (size_t)C * 2);
            continue;
        }
        if (t == 2) {
            float mn = orc_bf16_to_f32(row[0]), mx = mn;
            for (int64_t c = 1; c < C; ++c) {
                const float v = orc_bf16_to_f32(row[c]);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            float range = mx - mn;
            if (range < RANGE_FLOOR) range = RANGE_FLOOR;
            const float sc = range / 255.0f;
            const int z = (int)clampd((double)rintf(-128.0f - mn / sc), -128.0, 127.0);
            s8[k] = sc;
            z8[k] = (int8_t)z;
            for (int64_t c = 0; c < C; ++c)
                q8[k * C + c] = (int8_t)clampd((double)rintf(orc_bf16_to_f32(row[c]) / sc) + (double)z, -128.0, 127.0);
            continue;
        }
        const int qmax = t == 0 ? 1 : 7;
        float absmax = 0.0f;
        for (int64_t c = 0; c < C; ++c) {
            const float a = fabsf(orc_bf16_to_f32(row[c]));
            if (a > absmax) absmax = a;
        }
        if (absmax < RANGE_FLOOR) absmax = RANGE_FLOOR;
        const float sc = absmax / (float)qmax;
        if (t == 0) {
            s2[k] = sc;
            memset(&q2[k * (C / 4)], 0, (size_t)(C / 4));
        } else {
            s4[k] = sc;
            memset(&q4[k * (C / 2)], 0, (size_t)(C / 2));
        }
        for (int64_t c = 0; c < C; ++c) {
            const int q = (int)clampd((double)rintf(orc_bf16_to_f32(row[c]) / sc), -qmax, qmax);
            if (t == 0) q2[k * (C / 4) + c / 4] |= (uint8_t)((q & 3) << (2 * (c % 4)));
            else q4[k * (C / 2) + c / 2] |= (uint8_t)((q & 15) << (4 * (c % 2)));
        }
    }
    return 0;
}

/* x_hat = q * scale (2, 4 bits), (q - zero_point) * scale (8 bits), the bf16 value (16 bits);
 * fp32 out [N][C]. */
void orc_mixed_dequant(int64_t N, int64_t C, const uint8_t* tags, const int32_t* slot,
                       const uint8_t* q2, const float* s2, const uint8_t* q4, const float* s4,
                       const int8_t* q8, const float* s8, const int8_t* z8, const uint16_t* x16, float* out) {
    for (int64_t r = 0; r < N; ++r) {
        const int t = tag_of(tags, r);
        const int64_t k = slot[r];
        for (int64_t c = 0; c < C; ++c) {
            float v;
            if (t == 3) {
                v = orc_bf16_to_f32(x16[k * C + c]);
            } else if (t == 2) {
                v = ((float)q8[k * C + c] - (float)z8[k]) * s8[k];
            } else if (t == 1) {
                int q = (q4[k * (C / 2) + c / 2] >> (4 * (c % 2))) & 15;
                if (q >= 8) q -= 16;
                v = (float)q * s4[k];
            } else {
                int q = (q2[k * (C / 4) + c / 4] >> (2 * (c % 4))) & 3;
                if (q >= 2) q -= 4;
                v = (float)q * s2[k];
            }
            out[r * C + c] = v;
        }
    }
}

/* Bytes of a mixed-precision store: codes + scales (+ zero points) per pool, 16-bit rows, and
 * the 2-bit tags; out[0] = data, out[1] = scales and zero points, out[2] = tags. */
void orc_mixed_bytes(const int64_t counts[4], int64_t N, int64_t C, uint64_t out[3]) {
    out[0] = (uint64_t)(counts[0] * (C / 4) + counts[1] * (C / 2) + counts[2] * C + counts[3] * C * 2);
    out[1] = (uint64_t)(counts[0] * 4 + counts[1] * 4 + counts[2] * 5);
    out[2] = (uint64_t)((N + 3) / 4);
}

/* ------------------------------------------------------------ accounting --- */

/* [Explainer, group-size table] bytes = ceil(N/2) + ceil(N/g) * 4. */
uint64_t orc_int4_bytes(uint64_t N, uint64_t g) { return (N + 1) / 2 + ((N + g - 1) / g) * 4; }

int orc_int4_cache_sizes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, int64_t R,
                         uint64_t sect[8], uint64_t* total) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || d % 2 || g <= 0 || d % g || R < 0 || R > T) return -1;
    const uint64_t Tq = (uint64_t)(T - R), bh = (uint64_t)(B * H);
    sect[0] = bh * Tq * (uint64_t)(d / 2);                    /* K codes */
    sect[1] = bh * (uint64_t)ceil_div((int64_t)Tq, g) * (uint64_t)d * 2; /* K scales */
    sect[2] = sect[1];                                         /* K zeros */
    sect[3] = sect[0];                                         /* V codes */
    sect[4] = bh * Tq * (uint64_t)(d / g) * 2;                 /* V scales */
    sect[5] = sect[4];                                         /* V zeros */
    sect[6] = bh * (uint64_t)R * (uint64_t)d * 2;              /* K residual */
    sect[7] = sect[6];                                         /* V residual */
    uint64_t s = 0;
    for (int i = 0; i < 8; ++i) s += sect[i];
    *total = s;
    return 0;
}

/* [Walkthrough §2] original bytes / (data + scale + zero_point bytes). */
double orc_compression_ratio(uint64_t orig, uint64_t data, uint64_t scale, uint64_t zp) {
    return (double)orig / (double)(data + scale + zp);
}

/* [Walkthrough §4] T / K, rejected unless 0 < K <= T. */
int orc_token_ratio(int64_t T, int64_t K, double* out) {
    if (T <= 0 || K <= 0 || K > T) return -1;
    *out = (double)T / (double)K;
    return 0;
}

/* [Walkthrough §4] total gain ~ (s_old / s_new) * (T / K). */
double orc_total_gain(double s_old, double s_new, int64_t T, int64_t K) {
    return (s_old / s_new) * ((double)T / (double)K);
}

/* [Explainer, "four kinds of smaller" section] M ~ L * T_stored * C_stored * b + metadata. */
uint64_t orc_kv_bytes(uint64_t L, uint64_t T, uint64_t C, uint64_t b, uint64_t metadata) {
    return L * T * C * b + metadata;
}
