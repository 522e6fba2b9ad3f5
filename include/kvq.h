/* kvq.h -- C ABI of libkvq, KV-cache compression on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [Walkthrough] "KV Compression 公式到源码对照", formula-to-code walkthrough of a
 *                 per-channel quantizer and an H2O / SnapKV sparsifier (§1.1-§4).
 *   [Explainer]   "KV cache 压缩：把历史装得更小", animated explainer of KV-cache
 *                 compression: KIVI-style 4-bit groups, byte budgets, eviction,
 *                 fused dequantization in the attention kernel.
 *
 * Conventions shared by every entry point
 *   - Return value: KVQ_OK (0) or a negative status.  kvq_last_error() returns a
 *     thread-local description of the last failure of the calling thread.
 *   - Arguments are validated before anything is launched; on KVQ_EINVAL or
 *     KVQ_EALIGN nothing is written and nothing is enqueued.
 *   - Pointers named dev_* or documented as "device" are device (HBM) pointers;
 *     everything else is host memory.  The caller owns and allocates every
 *     buffer, including workspaces sized by the matching *_ws() query.  The
 *     library never allocates device memory.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t; NULL
 *     is the null stream); no entry point synchronizes the host.
 *   - Device pointers must be 16-byte aligned; innermost dimensions are dense.
 *   - bf16 data are raw 16-bit patterns (uint16_t).  fp32 -> bf16 rounds to
 *     nearest even.
 *   - Inputs are finite.  Codes, scales, zero points, packed bytes and kept
 *     indices are bit-identical to the plain definitions given below (fp32 IEEE
 *     division, round-half-to-even, no fused steps).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_OK 0
#define KVQ_EINVAL (-1) /* a shape, size or parameter the operation does not define */
#define KVQ_EALIGN (-2) /* a device pointer is not 16-byte aligned */
#define KVQ_EHIP (-3)   /* the HIP runtime reported an error (launch, stream) */

#define KVQ_FP32 0
#define KVQ_BF16 1

typedef void* kvq_stream; /* hipStream_t */

const char* kvq_last_error(void);
int kvq_abi_version(void); /* 1 */

/* ======================================================================
 * Per-channel quantization  [Walkthrough §1.1, §1.2]
 *
 * x holds nb slices, each a [R][C] matrix (rows = tokens, columns = channels;
 * a multi-dimensional cache puts every non-token dimension into C).  Element
 * (s, r, c) is at x + s*bsx + r*ldx + c (in elements of type xt).  Channel c of
 * slice s is quantized with its own scale, reduced over the R rows.
 *
 * kvq_quant_sym:   qmax = 2^(bits-1) - 1, bits in [2, 8];
 *                  scale = max(max_r |x|, fp32(1e-8)) / qmax;
 *                  q = clip(round(x / scale), -qmax, qmax).
 * kvq_quant_asym:  scale = max(max_r x - min_r x, fp32(1e-8)) / (qmax - qmin);
 *                  zp = round(qmin - min_r x / scale) saturated to int8;
 *                  q = clip(round(x / scale) + zp, qmin, qmax); -128 <= qmin < qmax <= 127.
 * round() is round-half-to-even.
 *
 * Outputs (device): q int8 [nb][R][C] dense; scale fp32 [nb][C]; zp int8 [nb][C]
 * (zp is optional for sym and then filled with 0 when given).
 * Workspace (device): kvq_quant_pc_ws(nb, R, C) bytes.
 * EINVAL: nb, R or C < 1; ldx < C; bsx < R*ldx (when nb > 1); bits or qmin/qmax
 *         outside the ranges above; NULL x, q or scale (or zp for asym); a
 *         workspace smaller than the query.
 * ====================================================================== */
size_t kvq_quant_pc_ws(int64_t nb, int64_t R, int64_t C);
int kvq_quant_sym(const void* x, int xt, int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx,
                  int bits, int8_t* q, float* scale, int8_t* zp_or_null, void* ws, size_t ws_bytes,
                  kvq_stream stream);
int kvq_quant_asym(const void* x, int xt, int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx,
                   int qmin, int qmax, int8_t* q, float* scale, int8_t* zp, void* ws, size_t ws_bytes,
                   kvq_stream stream);

/* ======================================================================
 * KIVI-style 4-bit group quantization of one layer  [Explainer: quantization,
 * grouping axis, group-size table and residual-budget sections; integer steps of
 * Walkthrough §1.2 with qmin = 0, qmax = 15]
 *
 * Inputs K, V: bf16 [B][T][H][d] (device).  The first Tq = T - R tokens are
 * quantized, the last R tokens are kept verbatim as a bf16 residual.
 *   K is grouped per channel across g consecutive tokens (the last group of a
 *   channel is partial when g does not divide Tq); V is grouped per token across
 *   g consecutive channels.  Per group:
 *     s = smallest bf16 >= max(max(max - min, fp32(1e-8)) / 15, |min| / 256)
 *         (stored bf16; the second bound only binds for a group far from zero
 *         relative to its range, and makes z below an integer bf16 holds exactly)
 *     z = round(0 - min / s), stored as bf16 (|z| <= 256, exact)
 *     q = clip(round(x / s) + z, 0, 15), using the stored s and z.
 *   Every value is then within s / 2 of its dequantized level.
 *   Dequantization: x_hat = (q - z) * s, rounded once (exact in fp32).
 * Sections (device, caller-allocated, sizes from kvq_int4_cache_sizes), with
 * Q = cap (or Tq when cap is 0) and P = rcap (or R when rcap is 0) rows per (b, h):
 *   [0] k_codes u8   [B][H][Q][d/2]  byte j = code(2j) | code(2j+1) << 4
 *   [1] k_scale bf16 [B][H][ceil(Q/g)][d]
 *   [2] k_zero  bf16 [B][H][ceil(Q/g)][d]
 *   [3] v_codes u8   [B][H][Q][d/2]
 *   [4] v_scale bf16 [B][H][Q][d/g]
 *   [5] v_zero  bf16 [B][H][Q][d/g]
 *   [6] k_res   bf16 [B][H][P][d]
 *   [7] v_res   bf16 [B][H][P][d]
 * Only the first Tq (resp. R) rows of each (b, h) are in use; cap and rcap let a
 * cache grow in place (kvq_int4_append).  With cap = rcap = 0 the sections are
 * dense.  Total bytes of the quantized region follow ceil(N/2) + ceil(N/g)*4 per
 * group axis [Explainer, group-size table].
 * EINVAL: any of B, T, H < 1; d not in {64, 128, 256}; g not in {32, 64, 128} or
 *         g > d; R < 0 or R > T; cap (when nonzero) < Tq or not a multiple of g;
 *         rcap (when nonzero) < R; a NULL section pointer of nonzero size.
 * ====================================================================== */
typedef struct {
    int64_t B, T, H, d, g, R;
    uint8_t* k_codes;
    uint16_t* k_scale;
    uint16_t* k_zero;
    uint8_t* v_codes;
    uint16_t* v_scale;
    uint16_t* v_zero;
    uint16_t* k_res;
    uint16_t* v_res;
    int64_t cap;  /* quantized-token rows per (b, h) in the sections; 0: Tq (dense)  */
    int64_t rcap; /* residual rows per (b, h) in the sections; 0: R (dense)          */
} kvq_int4_cache;

int kvq_int4_cache_sizes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, int64_t R,
                         size_t sect_bytes[8], size_t* total);
int kvq_group_quant_int4(const void* K, const void* V, const kvq_int4_cache* c, kvq_stream stream);

/* ======================================================================
 * Streaming append (decode time)  [Explainer: residual-budget section -- the
 * newest tokens stay bf16; grouping-axis section -- a K group spans g tokens of a
 * channel, so it can only be quantized once g tokens have arrived]
 *
 * c: a growable cache (cap > 0, rcap > 0, both section layouts as above), with
 *    T - R a multiple of g (a batch-quantized prefix, or empty: T = R = 0).
 * k_new, v_new: bf16 [B][n][H][d] (device), 1 <= n <= g, the next n tokens.
 * The n tokens go after the residual.  When the residual then holds at least
 * r_keep + g tokens, its oldest g tokens are quantized -- K group (T - R) / g
 * and V rows T - R .. T - R + g - 1, exactly as kvq_group_quant_int4 would --
 * and the residual drops them (its rows move down by g).  Updates c->T and
 * c->R on the host.  Afterwards the cache equals kvq_group_quant_int4 of all T
 * tokens with the new R.  Needs rcap >= R + n and, on a flush, cap >= T - R + g;
 * rcap >= r_keep + 2g - 1 always suffices.  Asynchronous on the stream; the
 * sections must not be read by other work until it completes.
 * EINVAL: NULL pointers; cap or rcap 0; T - R or cap not a multiple of g;
 *         n outside [1, g]; R >= r_keep + g; capacity exceeded; shapes as above.
 * ====================================================================== */
int kvq_int4_append(kvq_int4_cache* c, const void* k_new, const void* v_new, int64_t n, int64_t r_keep,
                    kvq_stream stream);

/* ======================================================================
 * Eviction on a 4-bit cache  [Explainer: eviction section (only the selected KV
 * is kept) on the layout of its grouping-axis and residual-budget sections;
 * Walkthrough §4: the token saving multiplies the byte saving]
 *
 * keep: int32 [B][H][K] (device), for every (b, h) the tokens to keep, as indices
 * into the T tokens of src (the selectors' output with rows = B*H is one such
 * list).  dst (B, H, d, g of src; dst->T = K with 1 <= K <= src->T; dst->R = R2
 * with 0 <= R2 <= K; dense or growable) receives, per (b, h), the kept tokens in
 * keep order: the first K - R2 quantized, the last R2 as bf16.  With x the current
 * value of a kept token (its dequantized level, or its bf16 value):
 *   - a V row from the quantized part keeps its codes, scale and zero;
 *   - a new K group (g consecutive kept tokens; the last may be partial) whose
 *     tokens are exactly all tokens of one old K group, in order, keeps that
 *     group's codes, scales and zeros; every other new K group, and every V row
 *     of a kept bf16 token, is quantized from x as in kvq_group_quant_int4;
 *   - a new bf16 row is x rounded to nearest even.
 * Keeping every token with R2 = src->R reproduces src.  Indices outside [0, T)
 * are clamped into it (unspecified result, no out-of-bounds access).  No dst
 * section may overlap a src section (checked).  Asynchronous on the stream.
 * EINVAL: shapes as in kvq_group_quant_int4 for src and dst; mismatched B, H, d,
 *         g; dst->T > src->T; NULL keep; overlapping sections.
 * ====================================================================== */
int kvq_int4_evict(const kvq_int4_cache* src, const int32_t* keep, const kvq_int4_cache* dst, kvq_stream stream);

/* ======================================================================
 * Hadamard-rotated per-token 4-bit cache  [KV-COBRA notes (papernotes.org),
 * item 4: an orthogonal Walsh-Hadamard matrix with a fixed random sign flip
 * spreads every coordinate to the mean variance before scalar quantization;
 * the QuaRot / TurboQuant comparison: rotation removes outliers.  Group steps
 * as kvq_group_quant_int4 (Explainer, quantization section).]
 *
 * For every token and head, K and V rows are rotated,
 *   y = (1/sqrt(d)) * H_d * (s (.) x),   H_d the Sylvester Hadamard matrix,
 * with the caller's signs s (k_signs for K, v_signs for V: HOST arrays of d
 * int8 entries, each +1 or -1; the method's random draw).  The transform is
 * fp32 butterflies in a fixed order: stage h = 1, 2, 4, ..., d/2, pair
 * (j, j + h) with j & h == 0 -> (a + b, a - b); then one multiply by
 * fp32(1/sqrt(d)).  Every token is then quantized per token in groups of g
 * consecutive rotated coordinates (s, z, q as in kvq_group_quant_int4).  There
 * is no bf16 window: a per-token group does not wait for later tokens.
 * Sections (device, caller-allocated, sizes from kvq_rot_cache_sizes):
 *   [0] k_codes u8 [B][H][T][d/2] (low nibble = even coordinate)
 *   [1] k_scale, [2] k_zero bf16 [B][H][T][d/g]
 *   [3] v_codes, [4] v_scale, [5] v_zero likewise.
 * kvq_rot_dequant: one side (0 = K, 1 = V) back to the original coordinates,
 *   the levels (q - z) * s, then the inverse rotation s (.) ((1/sqrt(d)) H_d y)
 *   in the same fp32 order; out [B][T][H][d] of type ot.
 * kvq_rot_decode_attn: GQA decode attention in the rotated space: q' = R_K q
 *   (fp32), softmax over all T tokens of sm_scale * q' . k'_t (k' the rotated
 *   levels), o' = sum_t p_t v'_t, out = R_V^-1 o' (fp32, then ot).  Since R_K
 *   is orthogonal this is attention over the dequantized cache.  Head map and
 *   output types as kvq_decode_attn_int4; workspace kvq_rot_decode_attn_ws().
 * EINVAL: B, T, H < 1; d not in {64, 128, 256}; g not in {32, 64, 128} or
 *   g > d; B*T*H >= 2^31; NULL pointers; signs other than +-1; side / ot / Hq
 *   as above; short workspace.  EALIGN: device pointers not 16-byte aligned.
 * ====================================================================== */
typedef struct {
    int64_t B, T, H, d, g;
    uint8_t* k_codes;
    uint16_t* k_scale;
    uint16_t* k_zero;
    uint8_t* v_codes;
    uint16_t* v_scale;
    uint16_t* v_zero;
} kvq_rot_cache;

int kvq_rot_cache_sizes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, size_t sect_bytes[6], size_t* total);
int kvq_rot_quant_int4(const void* K, const void* V, const int8_t* k_signs, const int8_t* v_signs,
                       const kvq_rot_cache* c, kvq_stream stream);
int kvq_rot_dequant(const kvq_rot_cache* c, int side, const int8_t* signs, void* out, int ot, kvq_stream stream);
size_t kvq_rot_decode_attn_ws(const kvq_rot_cache* c, int64_t Hq);
int kvq_rot_decode_attn(const kvq_rot_cache* c, const int8_t* k_signs, const int8_t* v_signs, const void* q,
                        int64_t Hq, float sm_scale, void* out, int ot, void* ws, size_t ws_bytes, kvq_stream stream);

/* ======================================================================
 * Per-token mixed precision  [Adaptive-bit blog: §2.1 four precision levels,
 * 2/4/8/16 bits, chosen per token by a controller; §3.1 per-token dynamic
 * quantization, symmetric at 2 and 4 bits, asymmetric at 8 bits; §3.2 2-bit
 * precision tags 00/01/10/11 = 2/4/8/16 bits, tokens of one precision stored
 * contiguously.  Steps of Walkthrough §1.1 / §1.2 over a row.]
 *
 * The store holds N rows of C channels (a row is one token: the caller decides
 * whether it spans one head, C = d, or all heads, C = H*d).  The controller that
 * picks the widths is not part of this library: tags are given, packed four to a
 * byte, row r in bits 2(r%4), 2(r%4)+1 of tags[r/4] (device).
 *   tag 0, 2 bits, tag 1, 4 bits: qmax = 1 / 7; scale = max(max|x|, fp32(1e-8)) / qmax;
 *     q = clip(round(x / scale), -qmax, qmax); x_hat = q * scale.
 *   tag 2, 8 bits: scale = max(max x - min x, fp32(1e-8)) / 255;
 *     zp = round(-128 - min x / scale) saturated to int8;
 *     q = clip(round(x / scale) + zp, -128, 127); x_hat = (q - zp) * scale.
 *   tag 3, 16 bits: the bf16 row itself.
 * round() is round-half-to-even of the IEEE fp32 quotient; scales fp32.
 * kvq_mixed_plan: slot[r] = number of rows before r with the same tag (int32, device)
 *   and counts[4] = rows per tag (int64, device); workspace kvq_mixed_plan_ws(N).
 * Pools (device, caller-allocated, cap[t] rows each, usually the counts):
 *   q2 u8 [cap0][C/4] (2-bit two's complement, channel 4j+i in bits 2i..2i+1 of byte j),
 *   s2 fp32 [cap0]; q4 u8 [cap1][C/2] (4-bit two's complement, even channel low), s4 fp32 [cap1];
 *   q8 int8 [cap2][C], s8 fp32 [cap2], z8 int8 [cap2]; x16 bf16 [cap3][C].
 * kvq_mixed_quant: x bf16 [N][C] (device) -> row r at slot[r] of its tag's pool.
 * kvq_mixed_dequant: out [N][C] of type ot (fp32, or bf16 = RNE of the fp32 value).
 * A row whose slot is outside [0, cap) of its pool is skipped (dequant writes 0).
 * kvq_mixed_bytes (host): out[0] codes + 16-bit rows, out[1] scales + zero points,
 *   out[2] tag bytes, for given counts.
 * EINVAL: N < 1 or N >= 2^31; C not a power of two in [64, 8192]; NULL tags, slot,
 *   counts or a needed pool; negative capacities; short workspace.
 * ====================================================================== */
typedef struct {
    int64_t N, C;
    const uint8_t* tags;
    const int32_t* slot;
    int64_t cap[4];
    uint8_t* q2;
    float* s2;
    uint8_t* q4;
    float* s4;
    int8_t* q8;
    float* s8;
    int8_t* z8;
    uint16_t* x16;
} kvq_mixed_store;

size_t kvq_mixed_plan_ws(int64_t N);
int kvq_mixed_plan(const uint8_t* tags, int64_t N, int32_t* slot, int64_t* counts, void* ws, size_t ws_bytes,
                   kvq_stream stream);
int kvq_mixed_quant(const void* x, const kvq_mixed_store* m, kvq_stream stream);
int kvq_mixed_dequant(const kvq_mixed_store* m, void* out, int ot, kvq_stream stream);
int kvq_mixed_bytes(const int64_t counts[4], int64_t N, int64_t C, uint64_t out[3]);

/* ======================================================================
 * Dequantization  [Walkthrough §1.3: x_hat = (q - zero_point) * scale]
 *
 * kind KVQ_FMT_PER_CHANNEL: desc -> kvq_pc_tensor; out [nb][R][C] dense.
 *      x_hat = ((float)(q - zp)) * scale, one fp32 rounding (zp NULL = 0).
 * kind KVQ_FMT_INT4_K / KVQ_FMT_INT4_V: desc -> kvq_int4_cache; out is the
 *      original [B][T][H][d] layout of K (resp. V); residual tokens are copied.
 * ot: KVQ_FP32 or KVQ_BF16 (fp32 result rounded to nearest even).
 * EINVAL: unknown kind or ot, NULL pointers, shapes as for the quantizers.
 * ====================================================================== */
#define KVQ_FMT_PER_CHANNEL 1
#define KVQ_FMT_INT4_K 2
#define KVQ_FMT_INT4_V 3

typedef struct {
    const int8_t* q;
    const float* scale;
    const int8_t* zp; /* may be NULL */
    int64_t nb, R, C;
} kvq_pc_tensor;

typedef struct {
    int kind;
    const void* desc;
} kvq_qdesc;

int kvq_dequant(const kvq_qdesc* src, void* out, int ot, kvq_stream stream);

/* ======================================================================
 * Error statistics  [Walkthrough §1.3: RMSE, max_abs_error, mean_abs_error]
 *
 * dev_out (device, 3 doubles, 8-byte aligned): sum (x - x_hat)^2, sum |x - x_hat|, max |x - x_hat|
 * over n elements, accumulated in fp64 with a fixed (run-to-run identical) order.
 * kvq_stats_finalize (host): rmse = sqrt(sum_sq / n), mean = sum_abs / n.
 * Workspace (device): kvq_err_stats_ws(n) bytes.
 * EINVAL: n < 1, NULL pointers, unknown dtypes, short workspace.
 * ====================================================================== */
size_t kvq_err_stats_ws(int64_t n);
int kvq_err_stats(const void* x, int xt, const void* xhat, int ht, int64_t n, double* dev_out,
                  void* ws, size_t ws_bytes, kvq_stream stream);
int kvq_stats_finalize(const double in[3], int64_t n, double* rmse, double* max_abs, double* mean_abs);

/* Host-only accounting helpers (pure functions, no device access). */
/* [Walkthrough §2] orig / (data + scale + zero_point); 0 when the denominator is 0. */
double kvq_compression_ratio(uint64_t orig_bytes, uint64_t data, uint64_t scale, uint64_t zp);
/* [Explainer, group-size table] ceil(N/2) + ceil(N/g) * 4; 0 when g == 0. */
uint64_t kvq_int4_bytes(uint64_t N, uint64_t g);
/* [Walkthrough §4] T / K; KVQ_EINVAL unless 0 < K <= T. */
int kvq_token_ratio(int64_t T, int64_t K, double* out);
/* [Walkthrough §4] (s_old / s_new) * (T / K); KVQ_EINVAL unless 0 < K <= T and s_new > 0. */
int kvq_total_gain(double s_old, double s_new, int64_t T, int64_t K, double* out);
/* [Explainer, section on the four ways to shrink the cache] L * T_stored * C_stored * b + metadata. */
uint64_t kvq_kv_bytes(uint64_t L, uint64_t T, uint64_t C, uint64_t b, uint64_t metadata);
/* [Walkthrough §3.2] size of recent ∪ TopK: min(T, max(budget, min(window, T))); -1 on bad input. */
int64_t kvq_keep_count(int64_t T, int64_t budget, int64_t window);

/* ======================================================================
 * GQA decode attention over the INT4 cache  [Explainer, quantization section
 * (dequantization inside the attention kernel) and evaluation section (fused
 * dequantization over a compact layout); GQA head sharing from the GQA section]
 *
 * For every batch b and query head hq (one query token each):
 *   h = hq / (Hq / H)   (consecutive query heads share a KV head)
 *   out[b][hq] = softmax_t(sm_scale * q[b][hq] . k_hat[b][t][h]) . v_hat[b][t][h]
 * over all T tokens: the INT4 tokens dequantized as in kvq_group_quant_int4 and
 * the R residual tokens read as bf16.  Scores, softmax and accumulation are fp32.
 * q is bf16 [B][Hq][d] (device); out is [B][Hq][d] (device) of type ot: KVQ_FP32, or
 * KVQ_BF16 = the fp32 result rounded to nearest even.
 * Workspace (device): kvq_decode_attn_int4_ws(c, Hq) bytes.
 * EINVAL: cache shape as above, Hq < 1, Hq % H != 0, Hq / H not in {1, 2, 4, 8, 16},
 *         unknown ot, NULL pointers, short workspace.
 * ====================================================================== */
size_t kvq_decode_attn_int4_ws(const kvq_int4_cache* c, int64_t Hq);
int kvq_decode_attn_int4(const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out,
                         int ot, void* ws, size_t ws_bytes, kvq_stream stream);

/* ======================================================================
 * Decode attention without a workspace  [for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops]
 *
 * The same operation, arguments and result as kvq_decode_attn_int4 (bit for bit), with the
 * split partials kept in a scratch array of KVQ_ATTN_SCRATCH_BYTES that the library holds
 * on each GPU it runs on, from its load until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating routine); its first call on a device takes the
 * array's address on that device.  Nothing in the scratch has to start at zero.  Every call
 * on a GPU shares that GPU's array: calls that overlap in time on one GPU (other streams,
 * other host threads) race and corrupt each other's output -- serialize them.
 * EINVAL: as kvq_decode_attn_int4, and kvq_decode_attn_int4_ws(c, Hq) above
 *         KVQ_ATTN_SCRATCH_BYTES (checked before anything is launched).
 * EHIP: the device or the scratch address could not be queried.
 * ====================================================================== */
#define KVQ_ATTN_SCRATCH_BYTES (16u << 20)
int kvq_decode_attn_int4_noalloc(const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out,
                                 int ot, kvq_stream stream);

/* ======================================================================
 * Decode attention with running H2O scores  [Walkthrough §3.1: a token's score
 * is the attention it has received, summed over the observed steps; applied one
 * decode step at a time; the attention itself as kvq_decode_attn_int4]
 *
 * out as kvq_decode_attn_int4 (bit for bit).  In addition, for every b, KV head h
 * and token t < T:
 *   acc[b][h][t] += sum over the Hq/H query heads hq of h (in hq order, fp32) of
 *                   p[b][hq][t] = softmax weight of token t in row (b, hq),
 * one fp32 addition per element.  acc: fp32 (device), row (b, h) at acc +
 * (b*H + h) * ld_acc; elements t >= T are not touched, so a caller can keep one
 * array for a growing cache (ld_acc = capacity) and evict with its rows.
 * Workspace (device): kvq_decode_attn_int4_h2o_ws(c, Hq) bytes (the attention's,
 * plus the per-token logits of every query head and each row's softmax max and sum).
 * EINVAL: as kvq_decode_attn_int4; NULL acc; ld_acc < T.  EALIGN: acc not 16-byte aligned.
 * ====================================================================== */
size_t kvq_decode_attn_int4_h2o_ws(const kvq_int4_cache* c, int64_t Hq);
int kvq_decode_attn_int4_h2o(const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out, int ot,
                             float* acc, int64_t ld_acc, void* ws, size_t ws_bytes, kvq_stream stream);

/* ======================================================================
 * H2O / SnapKV token selection  [Walkthrough §3.1-§3.3]
 *
 * kvq_h2o_select: hist fp32 [rows][T_obs][T] (device).  score[j] = sum over t of
 *   hist[t][j], fp32, added in t order from 0.0 (cumulative attention).  When
 *   scores_or_null is given the scores are also written there ([rows][T]).
 * kvq_snapkv_select: scores fp32 [rows][T] given (one-shot observation scores).
 * Both then, per row: recent = [max(0, T - window), T); the recent scores are
 *   replaced by -inf; TopK of the masked scores with k = max(0, budget - |recent|)
 *   (larger first, equal scores -> lower index, NaN below every number, and the
 *   recent tokens below every earlier token, NaN included, so the union always holds
 *   kvq_keep_count tokens); keep =
 *   the sorted union of recent and TopK, int32 [rows][kvq_keep_count(T, budget,
 *   window)] (device); when that count is 0, keep may be NULL and nothing is selected.
 * Workspace (device): kvq_select_ws(rows, T) bytes (h2o needs room for the scores
 *   when scores_or_null is NULL; snapkv needs none).
 * EINVAL: rows, T_obs or T < 1, T > 2^31 - 1, budget < 0, window < 0, NULL
 *   pointers, short workspace.
 * ====================================================================== */
size_t kvq_select_ws(int64_t rows, int64_t T);
int kvq_h2o_select(const float* hist, int64_t rows, int64_t T_obs, int64_t T, int64_t budget,
                   int64_t window, float* scores_or_null, int32_t* keep, void* ws, size_t ws_bytes,
                   kvq_stream stream);
int kvq_snapkv_select(const float* scores, int64_t rows, int64_t T, int64_t budget, int64_t window,
                      int32_t* keep, void* ws, size_t ws_bytes, kvq_stream stream);

/* ======================================================================
 * Compaction of the kept rows  [Explainer, eviction section: only the selected
 * positions stay in the cache]
 *
 * k_dst[b][k][h][:] = k_src[b][keep[b][h][k]][h][:] (and the same for V when both
 * v pointers are given).  k_src, v_src bf16 [B][T][H][d]; keep int32 [B][H][K] with
 * entries in [0, T) (the output of the selectors with rows = B*H); dst [B][K][H][d].
 * All device.  An entry outside [0, T) is clamped into range on the device: the row
 * it yields is unspecified, but nothing outside k_src / v_src is read.
 * EINVAL: B, T, H, d or K < 1, K > T, d % 8 != 0, NULL k pointers, exactly one
 *   of v_src / v_dst NULL.
 * ====================================================================== */
int kvq_compact(const void* k_src, const void* v_src_or_null, int64_t B, int64_t T, int64_t H, int64_t d,
                const int32_t* keep, int64_t K, void* k_dst, void* v_dst_or_null, kvq_stream stream);

/* ======================================================================
 * Streaming bandwidth probe  [a measurement helper, not a step of the method]
 *
 * Moves read_bytes from src and write_bytes to dst with the 16-byte loads and stores
 * the kernels above use (non-temporal when nt != 0), so that a kernel's time can be
 * read against what this device sustains for the same read:write mix.  Each workgroup
 * moves one tile: every thread issues its loads, then stores a value that depends on
 * them.  The ratio read_bytes : write_bytes must be 1:0 (read only), 0:1 (write only),
 * 1:1, 2:1, 1:2, 32:9 (a bf16 -> 4-bit g=64 quantizer's mix) or 9:32 (its
 * dequantizer's).  depth (1, 2, 4 or 8) multiplies the mix's accesses per thread (1:1
 * at depth 4: four loads and four stores; 32:9 and 9:32 take depth 1 only); thread t of
 * workgroup u makes its i-th store the 16 bytes (a ^ i, a, a, a) at chunk
 * (u * nstores + i) * 256 + t, a = t for a write-only probe.  dst is always required: a
 * read-only probe stores at most 16 bytes there.  Both device.
 * EINVAL: another ratio, another depth, sizes not multiples of 16, nothing to move,
 *   NULL pointers.
 * ====================================================================== */
int kvq_bw_probe(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes, int nt, int depth,
                 kvq_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
