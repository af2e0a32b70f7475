/*
 * kv4_oracle.h -- CPU oracle for the KV4-RL hybrid decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  A plain, slow, single-purpose statement of what
 * the path computes, used to check the HIP library.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * source, header, table or constant with the library.
 *
 * All pointers are HOST pointers.  BF16 and FP16 values travel as uint16_t
 * bit patterns.  Layouts (one layer's cache):
 *   pages       uint8  [num_pages][Hkv][2176]   one block per (page, kv-head)
 *   side_codes  int8   [max_slots][Hkv][144][2][128]   (K row, then V row)
 *   side_scales uint16 [max_slots][Hkv][144][2]        FP16 scales
 */
#ifndef KV4_ORACLE_H
#define KV4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv4ref_cache {
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t max_slots;
  uint8_t *pages;
  int8_t *side_codes;
  uint16_t *side_scales;
  int32_t sink;   /* s protected leading positions (16; a multiple of 16) */
  int32_t window; /* w protected recent positions (128); s + w <= 144 */
} kv4ref_cache;

/* Optional integer intermediates of a decode step (any pointer may be NULL).
 *   qcodes [B][Hq][128]      INT8 codes of the rotated query
 *   qsum   [B][Hq]           sum of those codes
 *   qk     [B][Hq][max_ctx]  int32 Q.K dot for every attended position
 *                            (INT4 codes in the main region, INT8 side codes
 *                            in the protected region)
 *   pcode  [B][Hq][max_ctx]  uint8 P-operand code of every main position
 *   pv     [B][Hq][max_pages][128]  int32 integer P.V accumulators of the
 *                            main tile on logical page j (j >= s / 16) */
typedef struct kv4ref_debug {
  int8_t *qcodes;
  int32_t *qsum;
  int32_t *qk;
  uint8_t *pcode;
  int32_t *pv;
  int32_t max_ctx;
  int32_t max_pages;
} kv4ref_debug;

/* scalar rules, exposed for the pins */
uint16_t kv4ref_f32_to_f16(float x);
float kv4ref_f16_to_f32(uint16_t h);
uint16_t kv4ref_f32_to_bf16(float x);
float kv4ref_bf16_to_f32(uint16_t h);
void kv4ref_convert_f16(const float *x, uint16_t *h, int64_t n);
void kv4ref_convert_bf16(const float *x, uint16_t *h, int64_t n);
void kv4ref_fwht128(float *x, int64_t nvec);
void kv4ref_quant_int4(const float *x, uint8_t *codes, uint16_t *delta, uint16_t *offset,
                       int64_t nvec);
void kv4ref_quant_int8(const float *x, int8_t *codes, uint16_t *scale, int64_t nvec);
void kv4ref_quant_query(const float *x, int8_t *codes, float *scale, int32_t *sum,
                        int64_t nvec);
void kv4ref_exp2s(const float *y, float *e, int64_t n);
void kv4ref_exp2s_coeffs(float *c8);
float kv4ref_scale_log2(float softmax_scale);

/* cache writers */
int kv4ref_append(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v,
                  const int32_t *pos, const int32_t *slot, const int32_t *page_table,
                  int32_t pt_stride, int32_t B);
int kv4ref_prefill(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *slot,
                   const int32_t *page_table, int32_t pt_stride, int32_t nseq, int32_t nthreads);

/* one decode step; pv_exact=1 replaces the integer P.V rule by the FP64 sum
 * over dequantized values (the cache-representation reference) */
int kv4ref_decode(const kv4ref_cache *c, const uint16_t *q, const int32_t *ctx_len,
                  const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B,
                  int32_t Hq, float softmax_scale, int32_t pv_exact, double *out, double *lse,
                  const kv4ref_debug *dbg, int32_t nthreads);

/* Re-prefill attention: the chunk of query tokens of sequence s at positions
 * start[s] .. start[s]+n_s-1 (n_s = cu[s+1]-cu[s]), after their K/V were written;
 * token i attends [0, start[s]+i] under the protected set of the cache ending at
 * start[s]+n_s.  q, out [T][Hq][128], lse [T][Hq]; dbg indexed by token. */
int kv4ref_prefill_attention(const kv4ref_cache *c, const uint16_t *q, const int32_t *cu_seqlens,
                             const int32_t *start_pos, const int32_t *slot,
                             const int32_t *page_table, int32_t pt_stride, int32_t nseq, int32_t Hq,
                             float softmax_scale, int32_t pv_exact, double *out, double *lse,
                             const kv4ref_debug *dbg, int32_t nthreads);
/* The same for the (token, q-head) pairs th[i] = token * Hq + head only:
 * out [n][128], lse [n] (FP64). */
int kv4ref_prefill_attention_sampled(const kv4ref_cache *c, const uint16_t *q, const int32_t *cu_seqlens,
                                     const int32_t *start_pos, const int32_t *slot,
                                     const int32_t *page_table, int32_t pt_stride, int32_t nseq,
                                     int32_t Hq, float softmax_scale, int32_t n, const int64_t *th,
                                     double *out, double *lse, int32_t nthreads);

/* KV8 everywhere (INT8 comparison variant): paged pool
 * uint8 [num_pages][num_kv_heads][4160] = K codes int8 [16][128] (rotated) |
 * V codes int8 [128][16] | s_k FP16 [16] | s_v FP16 [16]. */
typedef struct kv8ref_cache {
  int32_t num_pages;
  int32_t num_kv_heads;
  uint8_t *pages;
} kv8ref_cache;

int kv8ref_append(const kv8ref_cache *c, const uint16_t *k, const uint16_t *v, const int32_t *pos,
                  const int32_t *page_table, int32_t pt_stride, int32_t B);
int kv8ref_prefill(const kv8ref_cache *c, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *page_table,
                   int32_t pt_stride, int32_t nseq, int32_t nthreads);
/* Every position through the protected path's arithmetic; dbg: qcodes, qsum, qk. */
int kv8ref_decode(const kv8ref_cache *c, const uint16_t *q, const int32_t *ctx_len,
                  const int32_t *page_table, int32_t pt_stride, int32_t B, int32_t Hq,
                  float softmax_scale, double *out, double *lse, const kv4ref_debug *dbg,
                  int32_t nthreads);

/* MXFP4 variant: the same cache (pages of 2176 B, side buffer, budget) with
 * the main region in OCP MXFP4: K codes [16][64] | V codes [128][8] | K scales
 * E8M0 [16][4] | V scales E8M0 [16][4]. */
int mxref_append(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v, const int32_t *pos,
                 const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B);
int mxref_prefill(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v,
                  const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *slot,
                  const int32_t *page_table, int32_t pt_stride, int32_t nseq, int32_t nthreads);
int mxref_decode(const kv4ref_cache *c, const uint16_t *q, const int32_t *ctx_len,
                 const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B,
                 int32_t Hq, float softmax_scale, double *out, double *lse, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
