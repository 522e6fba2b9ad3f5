/* kvq_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded CPU reference for the KV-cache compression hot
 * path.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code, header, table or helper with
 * the GPU library: it is written from the pages' formulas alone.
 *
 * Every function follows one passage of the pages (cited at the definition in
 * kvq_oracle.c).  Floating point: fp32 steps are evaluated in fp32 exactly as
 * written (one IEEE operation, one round-to-nearest-even per step; built with
 * -ffp-contract=off so no step is fused), fp64 where the pages leave the
 * precision open (error statistics, attention).
 *
 * bf16 values are passed as their raw 16-bit patterns (uint16_t).
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Per-channel symmetric / asymmetric quantization of nb slices of [R][C]
 * (rows = tokens, columns = channels).  x is fp32 (x_bf16 == 0) or bf16. */
int orc_quant_sym(const void* x, int x_bf16, int64_t nb, int64_t R, int64_t C, int bits,
                  int8_t* q, float* scale, int8_t* zp);
int orc_quant_asym(const void* x, int x_bf16, int64_t nb, int64_t R, int64_t C, int qmin, int qmax,
                   int8_t* q, float* scale, int8_t* zp);
/* x_hat = (q - zp) * scale, fp32 [nb][R][C]; zp may be NULL (all zero). */
void orc_dequant_pc(const int8_t* q, const float* scale, const int8_t* zp,
                    int64_t nb, int64_t R, int64_t C, float* out);

/* out[0] = sum (x - xh)^2, out[1] = sum |x - xh|, out[2] = max |x - xh|, fp64, sequential. */
void orc_err_stats(const void* x, int x_bf16, const void* xh, int xh_bf16, int64_t n, double out[3]);
void orc_stats_finalize(const double in[3], int64_t n, double* rmse, double* max_abs, double* mean_abs);

/* KIVI-style 4-bit group quantization of one layer. K, V bf16 [B][T][H][d]. */
int orc_int4_quant(const uint16_t* K, const uint16_t* V, int64_t B, int64_t T, int64_t H, int64_t d,
                   int64_t g, int64_t R,
                   uint8_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                   uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                   uint16_t* k_res, uint16_t* v_res);
/* Dequantize one side (is_k = 1 for the per-channel K format, 0 for the per-token V format)
 * into fp32 [B][T][H][d]; residual rows are widened from bf16. */
void orc_int4_dequant(int is_k, const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                      const uint16_t* res, int64_t B, int64_t T, int64_t H, int64_t d, int64_t g,
                      int64_t R, float* out);

/* fp64 GQA decode attention over the dequantized INT4 cache. q bf16 [B][Hq][d]; out fp64 [B][Hq][d]. */
int orc_decode_attn(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                    const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                    const uint16_t* k_res, const uint16_t* v_res,
                    int64_t B, int64_t T, int64_t Hkv, int64_t d, int64_t g, int64_t R,
                    const uint16_t* q, int64_t Hq, double sm_scale, double* out);
/* Same, only for the listed (b, hq) rows: out [n_rows][d]; when probs is not NULL it also
 * receives each row's attention weights, fp64 [n_rows][T]. */
int orc_decode_attn_rows(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                         const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                         const uint16_t* k_res, const uint16_t* v_res,
                         int64_t B, int64_t T, int64_t Hkv, int64_t d, int64_t g, int64_t R,
                         const uint16_t* q, int64_t Hq, double sm_scale,
                         const int64_t* rows_b, const int64_t* rows_hq, int64_t n_rows, double* out,
                         double* probs);

/* H2O / SnapKV token selection. */
void orc_colsum(const float* hist, int64_t rows, int64_t T_obs, int64_t T, float* scores);
int64_t orc_keep_count(int64_t T, int64_t budget, int64_t window);
int orc_select(const float* scores, int64_t rows, int64_t T, int64_t budget, int64_t window, int32_t* keep);
int orc_h2o_select(const float* hist, int64_t rows, int64_t T_obs, int64_t T, int64_t budget,
                   int64_t window, float* scores, int32_t* keep);
void orc_compact(const uint16_t* src, int64_t B, int64_t T, int64_t H, int64_t d,
                 const int32_t* keep, int64_t K, uint16_t* dst);

/* Eviction on the 4-bit cache: keep int32 [B][H][K] (indices into the T tokens); the new
 * cache has K tokens, the last R2 of them bf16.  Destination layouts as orc_int4_quant. */
int orc_int4_evict(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                   const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                   const uint16_t* k_res, const uint16_t* v_res,
                   int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, int64_t R,
                   const int32_t* keep, int64_t K, int64_t R2,
                   uint8_t* dk_codes, uint16_t* dk_scale, uint16_t* dk_zero,
                   uint8_t* dv_codes, uint16_t* dv_scale, uint16_t* dv_zero,
                   uint16_t* dk_res, uint16_t* dv_res);

/* Hadamard-rotated per-token 4-bit cache.  signs: d entries in {+1, -1}. */
void orc_rotate_f32(const float* x, const int8_t* signs, int64_t n, int64_t d, float* y);
void orc_unrotate_f32(const float* y, const int8_t* signs, int64_t n, int64_t d, float* x);
int orc_rot_quant(const uint16_t* K, const uint16_t* V, int64_t B, int64_t T, int64_t H, int64_t d, int64_t g,
                  const int8_t* k_signs, const int8_t* v_signs,
                  uint8_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                  uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero);
void orc_rot_dequant(const uint8_t* codes, const uint16_t* scale, const uint16_t* zero, const int8_t* signs,
                     int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, float* out);
int orc_rot_decode_attn(const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                        const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                        const int8_t* k_signs, const int8_t* v_signs,
                        int64_t B, int64_t T, int64_t Hkv, int64_t d, int64_t g,
                        const uint16_t* q, int64_t Hq, double sm_scale, double* out);

/* Per-token mixed precision (tags packed four to a byte). */
void orc_mixed_plan(const uint8_t* tags, int64_t N, int32_t* slot, int64_t counts[4]);
int orc_mixed_quant(const uint16_t* x, int64_t N, int64_t C, const uint8_t* tags, const int32_t* slot,
                    uint8_t* q2, float* s2, uint8_t* q4, float* s4, int8_t* q8, float* s8, int8_t* z8,
                    uint16_t* x16);
void orc_mixed_dequant(int64_t N, int64_t C, const uint8_t* tags, const int32_t* slot,
                       const uint8_t* q2, const float* s2, const uint8_t* q4, const float* s4,
                       const int8_t* q8, const float* s8, const int8_t* z8, const uint16_t* x16, float* out);
void orc_mixed_bytes(const int64_t counts[4], int64_t N, int64_t C, uint64_t out[3]);

/* Accounting. */
uint64_t orc_int4_bytes(uint64_t N, uint64_t g);
int orc_int4_cache_sizes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t g, int64_t R,
                         uint64_t sect[8], uint64_t* total);
double orc_compression_ratio(uint64_t orig, uint64_t data, uint64_t scale, uint64_t zp);
int orc_token_ratio(int64_t T, int64_t K, double* out);
double orc_total_gain(double s_old, double s_new, int64_t T, int64_t K);
uint64_t orc_kv_bytes(uint64_t L, uint64_t T, uint64_t C, uint64_t b, uint64_t metadata);

/* bf16 helpers exposed for the tests (round to nearest even, widen). */
uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t b);
void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
