/*
 * kv4_oracle.c -- CPU oracle for the KV4-RL hybrid decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY (see kv4_oracle.h).  Plain, slow and written to be
 * read against the KV4-RL pages:
 *   - group-affine INT4 per 128-dim token-head vector, x^ = delta*c + m, FP16
 *     delta/m computed on line (paper.rainbus.top summary, "分组仿射 KV 量化",
 *     "方法步骤详情" step 2);
 *   - keys Hadamard-rotated after RoPE, queries given the same rotation, so
 *     that rotated scores equal the original ones (same sections);
 *   - INT8 copies of the first s=16 and the last w=128 positions in a fixed
 *     side buffer; leaving the window rewrites nothing in INT4 (step 3);
 *   - hybrid attention: rotated query quantized to INT8; main region integer
 *     QK and integer PV over unpacked INT4 codes with delta/m applied after
 *     the dot; protected region INT8 QK, BF16-dequantized V, FP32 PV; each
 *     region yields an output and a log-normalizer, merged exactly (step 4;
 *     onedev.kr summary, "전제와 한계").
 * Where the pages leave a step open the reading used is stated next to it.
 * Build: -O2 -fno-fast-math -ffp-contract=off (no silent FMA contraction).
 */
#include "kv4_oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum {
  HD = 128,          /* one quantization group = one 128-dim token-head vector */
  PAGE = 16,         /* positions per page */
  SIDE_ROWS = 144,   /* capacity of the side buffer per (slot, kv-head): s + w <= 144 */
  BLOCK = 2176,      /* bytes per (page, kv-head): 16 x (64+64+4+4) */
  OFF_KCODE = 0,     /* K codes, token-major, 64 B per position */
  OFF_VCODE = 1024,  /* V codes, channel-major, 8 B per channel */
  OFF_KMETA = 2048,  /* 16 x {delta, m} FP16 for K */
  OFF_VMETA = 2112   /* 16 x {delta, m} FP16 for V */
};

/* ------------------------------------------------------------------------ */
/* FP16 / BF16 round-to-nearest-even, written from the IEEE formats.          */
/* ------------------------------------------------------------------------ */

/* Round |a| (finite, non-zero) to a binary format with `mant` stored mantissa
 * bits and minimum normal exponent `emin`; returns the magnitude bits, or
 * UINT32_MAX on overflow past `emax`. */
static uint32_t round_binary(double a, int mant, int emin, int emax, int bias) {
  int e2;
  frexp(a, &e2);            /* a in [2^(e2-1), 2^e2) */
  int ex = e2 - 1;
  if (ex < emin) ex = emin; /* subnormals share the quantum of the lowest binade */
  double q = ldexp(a, mant - ex);  /* a / quantum, exact */
  double n = nearbyint(q);         /* ties to even (default rounding mode) */
  const double hidden = ldexp(1.0, mant);
  if (n >= 2.0 * hidden) {         /* carried into the next binade */
    n = hidden;
    ex += 1;
  }
  if (n < hidden) return (uint32_t)n;  /* subnormal (or zero) */
  if (ex > emax) return UINT32_MAX;
  return ((uint32_t)(ex + bias) << mant) | (uint32_t)(n - hidden);
}

uint16_t kv4ref_f32_to_f16(float x) {
  uint32_t bits;
  memcpy(&bits, &x, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(x)) return sign | 0x7e00u;
  if (isinf(x) || x == 0.0f) return sign | (isinf(x) ? 0x7c00u : 0u);
  uint32_t m = round_binary(fabs((double)x), 10, -14, 15, 15);
  if (m == UINT32_MAX) return sign | 0x7c00u;
  return sign | (uint16_t)m;
}

float kv4ref_f16_to_f32(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);
  return (float)(s ? -v : v);
}

uint16_t kv4ref_f32_to_bf16(float x) {
  uint32_t bits;
  memcpy(&bits, &x, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(x)) return sign | 0x7fc0u;
  if (isinf(x) || x == 0.0f) return sign | (isinf(x) ? 0x7f80u : 0u);
  uint32_t m = round_binary(fabs((double)x), 7, -126, 127, 127);
  if (m == UINT32_MAX) return sign | 0x7f80u;
  return sign | (uint16_t)m;
}

/* BF16 is the upper half of a binary32 pattern. */
float kv4ref_bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

void kv4ref_convert_f16(const float *x, uint16_t *h, int64_t n) {
  for (int64_t i = 0; i < n; i++) h[i] = kv4ref_f32_to_f16(x[i]);
}

void kv4ref_convert_bf16(const float *x, uint16_t *h, int64_t n) {
  for (int64_t i = 0; i < n; i++) h[i] = kv4ref_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Hadamard rotation (keys after RoPE, and the query).                        */
/* Reading: H = H_128 / sqrt(128) (Sylvester, orthonormal).  FP32 in-place    */
/* fast Walsh-Hadamard transform with strides 1, 2, ..., 64 in that order,    */
/* then every element is multiplied once by fp32(2^-3.5).                     */
/* ------------------------------------------------------------------------ */

static const float INV_SQRT128 = 0x1.6a09e6p-4f; /* fp32 RNE of 2^-3.5 */

static void fwht128(float x[HD]) {
  for (int h = 1; h < HD; h <<= 1) {
    for (int i = 0; i < HD; i++) {
      if (i & h) continue;
      float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
  for (int i = 0; i < HD; i++) x[i] = x[i] * INV_SQRT128;
}

void kv4ref_fwht128(float *x, int64_t nvec) {
  for (int64_t v = 0; v < nvec; v++) fwht128(x + v * HD);
}

/* ------------------------------------------------------------------------ */
/* Quantizers.                                                                */
/* ------------------------------------------------------------------------ */

static void check_domain(const float x[HD]) {
  for (int i = 0; i < HD; i++) assert(isfinite(x[i]) && fabsf(x[i]) <= 65504.0f);
}

/* Group-affine INT4: x^ = delta*c + m, FP16 delta and m, b = 4.
 * delta = fp16((max-min)/15) with FP32 min/max, FP32 subtraction and IEEE
 * division; reading: the offset m is fp16(min); c = clamp(rint((x-m)/delta),
 * 0, 15) in FP32 with ties to even; a zero delta gives all-zero codes. */
static void quant_int4(const float x[HD], uint8_t c[HD], uint16_t *delta16, uint16_t *m16) {
  check_domain(x);
  float mn = x[0], mx = x[0];
  for (int i = 1; i < HD; i++) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  float range = mx - mn;
  *delta16 = kv4ref_f32_to_f16(range / 15.0f);
  *m16 = kv4ref_f32_to_f16(mn);
  float d = kv4ref_f16_to_f32(*delta16);
  float m = kv4ref_f16_to_f32(*m16);
  for (int i = 0; i < HD; i++) {
    if (d == 0.0f) {
      c[i] = 0;
      continue;
    }
    float t = rintf((x[i] - m) / d);
    if (t < 0.0f) t = 0.0f;
    if (t > 15.0f) t = 15.0f;
    c[i] = (uint8_t)t;
  }
}

/* Reading of the INT8 side copy: symmetric per 128-vector, scale
 * s = fp16(max|x| / 127), c = clamp(rint(x / s), -127, 127); s = 0 gives
 * zero codes. */
static void quant_int8(const float x[HD], int8_t c[HD], uint16_t *s16) {
  check_domain(x);
  float a = 0.0f;
  for (int i = 0; i < HD; i++)
    if (fabsf(x[i]) > a) a = fabsf(x[i]);
  *s16 = kv4ref_f32_to_f16(a / 127.0f);
  float s = kv4ref_f16_to_f32(*s16);
  for (int i = 0; i < HD; i++) {
    if (s == 0.0f) {
      c[i] = 0;
      continue;
    }
    float t = rintf(x[i] / s);
    if (t < -127.0f) t = -127.0f;
    if (t > 127.0f) t = 127.0f;
    c[i] = (int8_t)t;
  }
}

/* Symmetric INT8 of the rotated query, FP32 scale (never stored, so never
 * rounded to FP16): s = max|x| / 127, c = clamp(rint(x / s), -127, 127),
 * s = 0 gives zero codes; also returns the code sum used by the deferred
 * offset term. */
static void quant_query(const float x[HD], int8_t c[HD], float *s_out, int32_t *sum) {
  float a = 0.0f;
  for (int i = 0; i < HD; i++)
    if (fabsf(x[i]) > a) a = fabsf(x[i]);
  float s = a / 127.0f;
  int32_t acc = 0;
  for (int i = 0; i < HD; i++) {
    if (s == 0.0f) {
      c[i] = 0;
      continue;
    }
    float t = rintf(x[i] / s);
    if (t < -127.0f) t = -127.0f;
    if (t > 127.0f) t = 127.0f;
    c[i] = (int8_t)t;
    acc += c[i];
  }
  *s_out = (s == 0.0f) ? 0.0f : s;
  *sum = acc;
}

void kv4ref_quant_int4(const float *x, uint8_t *codes, uint16_t *delta, uint16_t *offset,
                       int64_t nvec) {
  for (int64_t v = 0; v < nvec; v++)
    quant_int4(x + v * HD, codes + v * HD, delta + v, offset + v);
}

void kv4ref_quant_int8(const float *x, int8_t *codes, uint16_t *scale, int64_t nvec) {
  for (int64_t v = 0; v < nvec; v++) quant_int8(x + v * HD, codes + v * HD, scale + v);
}

void kv4ref_quant_query(const float *x, int8_t *codes, float *scale, int32_t *sum,
                        int64_t nvec) {
  for (int64_t v = 0; v < nvec; v++)
    quant_query(x + v * HD, codes + v * HD, scale + v, sum + v);
}

/* ------------------------------------------------------------------------ */
/* exp2 used for the softmax weights.  The pages say only "exact softmax      */
/* merge"; reading: a fixed evaluation both sides can reproduce bit for bit,  */
/* so that the P-operand codes and their integer accumulators are unique:     */
/* y < -125 -> 0; otherwise n = rint(y), f = y - n (exact), p = Taylor series */
/* of 2^f to degree 7 in Horner form with fmaf and coefficients               */
/* fp32(ln2^k / k!), result p * 2^n.                                          */
/* ------------------------------------------------------------------------ */

static float EXP2_C[8];
static int exp2_ready = 0;

static void exp2_init(void) {
  if (exp2_ready) return;
  double ln2 = log(2.0), term = 1.0;
  for (int k = 0; k < 8; k++) {
    EXP2_C[k] = (float)term;   /* ln2^k / k! */
    term = term * ln2 / (double)(k + 1);
  }
  exp2_ready = 1;
}

static float exp2s(float y) {
  if (!(y >= -125.0f)) return 0.0f;
  float n = rintf(y);
  float f = y - n;
  float p = EXP2_C[7];
  for (int k = 6; k >= 0; k--) p = fmaf(p, f, EXP2_C[k]);
  return ldexpf(p, (int)n);
}

void kv4ref_exp2s(const float *y, float *e, int64_t n) {
  exp2_init();
  for (int64_t i = 0; i < n; i++) e[i] = exp2s(y[i]);
}

void kv4ref_exp2s_coeffs(float *c8) {
  exp2_init();
  for (int k = 0; k < 8; k++) c8[k] = EXP2_C[k];
}

/* Softmax runs in base 2: logits carry softmax_scale * log2(e). */
float kv4ref_scale_log2(float softmax_scale) {
  return (float)((double)softmax_scale * M_LOG2E);
}

/* ------------------------------------------------------------------------ */
/* Cache layout (the pages only say "paged INT4"; reading):                   */
/*   block(page, kv-head) = K codes 1024 B (position t at bytes 64t..64t+63,  */
/*   channel 2i in the low nibble and 2i+1 in the high nibble of byte i) ||   */
/*   V codes 1024 B (channel j at bytes 8j..8j+7, position 2k in the low and  */
/*   2k+1 in the high nibble of byte k) || 16 x {delta, m} FP16 for K ||      */
/*   16 x {delta, m} FP16 for V (little-endian).  68 B per 128 elements:      */
/*   4.25 bits per element.                                                   */
/* Side rows (s sink positions, w recent positions; s = 16, w = 128 by       */
/* default): position p < s -> row p; p >= s -> row s + (p mod w), or no row */
/* when w = 0.                                                               */
/* ------------------------------------------------------------------------ */

static uint8_t *block_at(const kv4ref_cache *c, int32_t phys, int g) {
  assert(phys >= 0 && phys < c->num_pages);
  return c->pages + ((size_t)phys * (size_t)c->num_kv_heads + (size_t)g) * BLOCK;
}

/* Protection budget: s a multiple of the page size, s + w within the buffer. */
static int budget_ok(const kv4ref_cache *c) {
  return c->sink >= 0 && c->window >= 0 && c->sink % PAGE == 0 && c->sink + c->window <= SIDE_ROWS;
}

/* Side row of position p, or -1 when p has none (p >= s and w = 0). */
static int side_row(const kv4ref_cache *c, int32_t p) {
  if (p < c->sink) return p;
  return c->window > 0 ? c->sink + (p % c->window) : -1;
}

static int8_t *side_code_at(const kv4ref_cache *c, int32_t slot, int g, int row, int kv) {
  assert(slot >= 0 && slot < c->max_slots);
  size_t r = ((size_t)slot * (size_t)c->num_kv_heads + (size_t)g) * SIDE_ROWS + (size_t)row;
  return c->side_codes + (r * 2 + (size_t)kv) * HD;
}

static uint16_t *side_scale_at(const kv4ref_cache *c, int32_t slot, int g, int row, int kv) {
  size_t r = ((size_t)slot * (size_t)c->num_kv_heads + (size_t)g) * SIDE_ROWS + (size_t)row;
  return c->side_scales + r * 2 + (size_t)kv;
}

static void put_meta(uint8_t *blk, int off, int t, uint16_t delta, uint16_t m) {
  blk[off + 4 * t + 0] = (uint8_t)(delta & 0xff);
  blk[off + 4 * t + 1] = (uint8_t)(delta >> 8);
  blk[off + 4 * t + 2] = (uint8_t)(m & 0xff);
  blk[off + 4 * t + 3] = (uint8_t)(m >> 8);
}

static void get_meta(const uint8_t *blk, int off, int t, float *delta, float *m) {
  uint16_t d = (uint16_t)(blk[off + 4 * t] | (blk[off + 4 * t + 1] << 8));
  uint16_t o = (uint16_t)(blk[off + 4 * t + 2] | (blk[off + 4 * t + 3] << 8));
  *delta = kv4ref_f16_to_f32(d);
  *m = kv4ref_f16_to_f32(o);
}

static void put_k_codes(uint8_t *blk, int t, const uint8_t c[HD]) {
  for (int i = 0; i < HD / 2; i++)
    blk[OFF_KCODE + 64 * t + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
}

static void get_k_codes(const uint8_t *blk, int t, uint8_t c[HD]) {
  for (int i = 0; i < HD / 2; i++) {
    uint8_t byte = blk[OFF_KCODE + 64 * t + i];
    c[2 * i] = byte & 15;
    c[2 * i + 1] = byte >> 4;
  }
}

static void put_v_codes(uint8_t *blk, int t, const uint8_t c[HD]) {
  for (int j = 0; j < HD; j++) {
    uint8_t *byte = &blk[OFF_VCODE + 8 * j + t / 2];
    if (t % 2 == 0) *byte = (uint8_t)((*byte & 0xF0) | c[j]);
    else *byte = (uint8_t)((*byte & 0x0F) | (c[j] << 4));
  }
}

static uint8_t get_v_code(const uint8_t *blk, int t, int j) {
  uint8_t byte = blk[OFF_VCODE + 8 * j + t / 2];
  return (t % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* ------------------------------------------------------------------------ */
/* Quantize-on-append: every position goes to INT4; sink and recent          */
/* positions also get an INT8 row (the ring row of an evicted position is     */
/* simply overwritten; its INT4 entry stays).                                 */
/* ------------------------------------------------------------------------ */

static void append_one(const kv4ref_cache *c, int g, const uint16_t *k16, const uint16_t *v16,
                       int32_t pos, int32_t slot, const int32_t *table_row) {
  float k[HD], v[HD];
  for (int i = 0; i < HD; i++) {
    k[i] = kv4ref_bf16_to_f32(k16[i]);
    v[i] = kv4ref_bf16_to_f32(v16[i]);
  }
  fwht128(k); /* keys are stored in the rotated basis; values are not rotated */

  uint8_t kc[HD], vc[HD];
  uint16_t kd, km, vd, vm;
  quant_int4(k, kc, &kd, &km);
  quant_int4(v, vc, &vd, &vm);
  uint8_t *blk = block_at(c, table_row[pos / PAGE], g);
  int t = pos % PAGE;
  put_k_codes(blk, t, kc);
  put_v_codes(blk, t, vc);
  put_meta(blk, OFF_KMETA, t, kd, km);
  put_meta(blk, OFF_VMETA, t, vd, vm);

  int row = side_row(c, pos);
  if (row < 0) return;
  quant_int8(k, side_code_at(c, slot, g, row, 0), side_scale_at(c, slot, g, row, 0));
  quant_int8(v, side_code_at(c, slot, g, row, 1), side_scale_at(c, slot, g, row, 1));
}

int kv4ref_append(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v,
                  const int32_t *pos, const int32_t *slot, const int32_t *page_table,
                  int32_t pt_stride, int32_t B) {
  const int H = c->num_kv_heads;
  if (!budget_ok(c)) return -1;
  for (int b = 0; b < B; b++) {
    int32_t s = slot ? slot[b] : b;
    for (int g = 0; g < H; g++) {
      size_t off = ((size_t)b * H + g) * HD;
      append_one(c, g, k + off, v + off, pos[b], s, page_table + (size_t)b * pt_stride);
    }
  }
  return 0;
}

/* Re-prefill is defined as the appends of its tokens, in order. */
int kv4ref_prefill(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *slot,
                   const int32_t *page_table, int32_t pt_stride, int32_t nseq, int32_t nthreads) {
  const int H = c->num_kv_heads;
  (void)nthreads;
  if (!budget_ok(c)) return -1;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int sq = 0; sq < nseq; sq++) {
    int32_t s = slot ? slot[sq] : sq;
    for (int32_t i = 0; i < cu_seqlens[sq + 1] - cu_seqlens[sq]; i++) {
      size_t tok = (size_t)cu_seqlens[sq] + (size_t)i;
      for (int g = 0; g < H; g++) {
        size_t off = (tok * H + g) * HD;
        append_one(c, g, k + off, v + off, start_pos[sq] + i, s,
                   page_table + (size_t)sq * pt_stride);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode.                                                                    */
/* Regions (L = context length including this step's token; s = 16 and     */
/* w = 128 by default):                                                       */
/*   sinks  S = [0, min(s, L)),  recent R = [max(s, L-w), L),                 */
/*   main   M = [s, L-w)  (empty when L <= s + w).                            */
/* A partial is (A[128], Z, l): unnormalised output, base-2 max logit and sum */
/* of weights relative to Z.  Everything after the integer accumulators is    */
/* evaluated in FP64 here.                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  double A[HD];
  double Z;
  double l;
} partial_t;

/* Main-region P-operand rule, per tile = logical page intersected with M:
 *   z_max = max z_t; e_t = exp2s(z_t - z_max); u_t = e_t * delta_v(t);
 *   u_max = max u_t; uc_t = clamp(rint(u_t * (127 / u_max)), 0, 127) (FP32);
 *   acc_j = sum_t uc_t * cv(t, j) (exact integer);
 *   A_j = (u_max / 127) * acc_j + sum_t e_t * m_v(t);  l = sum_t e_t.
 * The per-position V scale is folded into P, which integer PV over positions
 * needs; the per-position V offset is channel-independent and applied after
 * the dot; normalisation uses the unquantized weights. */
static void main_tile(const uint8_t *blk, int t_end, const int8_t qc[HD], int32_t qsum, float c_q,
                      int pv_exact, partial_t *out, int32_t *dbg_qk, uint8_t *dbg_pc,
                      int32_t *dbg_pv) {
  float z[PAGE], e[PAGE], u[PAGE], dv[PAGE], mv[PAGE];
  for (int t = 0; t < t_end; t++) {
    uint8_t kc[HD];
    get_k_codes(blk, t, kc);
    int32_t D = 0;
    for (int i = 0; i < HD; i++) D += (int32_t)qc[i] * (int32_t)kc[i];
    float dk, mk;
    get_meta(blk, OFF_KMETA, t, &dk, &mk);
    /* q.k^ = s_q (delta * sum(qc*c) + m * sum(qc)); base-2 scale folded in c_q */
    z[t] = fmaf(dk, (float)D, mk * (float)qsum) * c_q;
    get_meta(blk, OFF_VMETA, t, &dv[t], &mv[t]);
    if (dbg_qk) dbg_qk[t] = D;
  }
  float zmax = -INFINITY; /* t_end >= 1 */
  for (int t = 0; t < t_end; t++)
    if (z[t] > zmax) zmax = z[t];
  float umax = 0.0f;
  for (int t = 0; t < t_end; t++) {
    e[t] = exp2s(z[t] - zmax);
    u[t] = e[t] * dv[t];
    if (u[t] > umax) umax = u[t];
  }
  out->Z = zmax;
  out->l = 0.0;
  double mu = 0.0;
  for (int t = 0; t < t_end; t++) {
    out->l += (double)e[t];
    mu += (double)e[t] * (double)mv[t];
  }
  if (pv_exact) {
    for (int j = 0; j < HD; j++) {
      double a = 0.0;
      for (int t = 0; t < t_end; t++)
        a += (double)e[t] * ((double)dv[t] * (double)get_v_code(blk, t, j) + (double)mv[t]);
      out->A[j] = a;
    }
    return;
  }
  int32_t uc[PAGE];
  float inv = (umax == 0.0f) ? 0.0f : 127.0f / umax;
  for (int t = 0; t < t_end; t++) {
    if (umax == 0.0f) {
      uc[t] = 0;
    } else {
      /* a u_max below 127 / FLT_MAX makes inv infinite: a zero weight then
       * gives 0 * inf = NaN, read as code 0, and every nonzero one 127 */
      float r = rintf(u[t] * inv);
      if (!(r >= 0.0f)) r = 0.0f;
      if (r > 127.0f) r = 127.0f;
      uc[t] = (int32_t)r;
    }
    if (dbg_pc) dbg_pc[t] = (uint8_t)uc[t];
  }
  double s_u = (double)umax / 127.0;
  for (int j = 0; j < HD; j++) {
    int32_t acc = 0;
    for (int t = 0; t < t_end; t++) acc += uc[t] * (int32_t)get_v_code(blk, t, j);
    if (dbg_pv) dbg_pv[j] = acc;
    out->A[j] = s_u * (double)acc + mu;
  }
}

/* INT8 rows of one region: position, key and value codes and FP16 scales. */
typedef struct {
  int32_t pos;
  const int8_t *k8, *v8;
  uint16_t sk, sv;
} int8_row_t;

/* The protected path's arithmetic over n INT8 rows: the INT8 query against
 * the INT8 keys, z = (D8 * s_k) * c_q; FP32 softmax weights relative to the
 * region max; values dequantized to BF16, v^ = bf16(s_v * c); P stays FP32. */
static void int8_region(const int8_row_t *rows, int n, const int8_t qc[HD], float c_q,
                        partial_t *out, int32_t *dbg_qk) {
  out->Z = -INFINITY; /* an empty region contributes nothing */
  out->l = 0.0;
  for (int j = 0; j < HD; j++) out->A[j] = 0.0;
  if (n == 0) return;
  float *z = (float *)malloc(sizeof(float) * (size_t)n);
  for (int i = 0; i < n; i++) {
    int32_t D8 = 0;
    for (int d = 0; d < HD; d++) D8 += (int32_t)qc[d] * (int32_t)rows[i].k8[d];
    z[i] = ((float)D8 * kv4ref_f16_to_f32(rows[i].sk)) * c_q;
    if (dbg_qk) dbg_qk[rows[i].pos] = D8;
  }
  float zmax = -INFINITY;
  for (int i = 0; i < n; i++)
    if (z[i] > zmax) zmax = z[i];
  out->Z = zmax;
  for (int i = 0; i < n; i++) {
    float e = exp2s(z[i] - zmax);
    float sv = kv4ref_f16_to_f32(rows[i].sv);
    out->l += (double)e;
    for (int j = 0; j < HD; j++) {
      float vhat = kv4ref_bf16_to_f32(kv4ref_f32_to_bf16(sv * (float)rows[i].v8[j]));
      out->A[j] += (double)e * (double)vhat;
    }
  }
  free(z);
}

/* Protected region of a query that attends [0, L) while the cache holds
 * positions [0, E) (E = L for a decode step): the sinks below L and the
 * window positions [max(s, E-w), L), read from the side rows. */
static void protected_region(const kv4ref_cache *c, int32_t slot, int g, int32_t L, int32_t E,
                             const int8_t qc[HD], float c_q, partial_t *out, int32_t *dbg_qk) {
  int32_t pos[SIDE_ROWS];
  int n = 0;
  const int sw = c->sink + c->window;
  int sink_end = L < c->sink ? L : c->sink;
  int rec_begin = (E - c->window) > c->sink ? (E - c->window) : c->sink;
  for (int p = 0; p < sink_end; p++) pos[n++] = p;
  for (int p = rec_begin; p < L; p++) pos[n++] = p;
  assert(n <= sw && (E != L || n == (L < sw ? L : sw)));
  int8_row_t rows[SIDE_ROWS];
  for (int i = 0; i < n; i++) {
    int row = side_row(c, pos[i]);
    rows[i].pos = pos[i];
    rows[i].k8 = side_code_at(c, slot, g, row, 0);
    rows[i].v8 = side_code_at(c, slot, g, row, 1);
    rows[i].sk = *side_scale_at(c, slot, g, row, 0);
    rows[i].sv = *side_scale_at(c, slot, g, row, 1);
  }
  int8_region(rows, n, qc, c_q, out, dbg_qk);
}

/* Exact log-sum-exp merge of region partials. */
static void merge(const partial_t *p, int n, double *out, double *lse) {
  double Z = -INFINITY;
  for (int r = 0; r < n; r++)
    if (p[r].Z > Z) Z = p[r].Z;
  double l = 0.0;
  double o[HD];
  for (int j = 0; j < HD; j++) o[j] = 0.0;
  for (int r = 0; r < n; r++) {
    if (p[r].l == 0.0) continue; /* empty region */
    double w = exp2(p[r].Z - Z);
    l += w * p[r].l;
    for (int j = 0; j < HD; j++) o[j] += w * p[r].A[j];
  }
  for (int j = 0; j < HD; j++) out[j] = o[j] / l;
  *lse = M_LN2 * (Z + log2(l));
}

/* One (query, q-head): attends [0, L) of the cache holding [0, E).  Main
 * region M = [s, min(L, E-w)); the rest as protected_region. */
static void decode_one_query(const kv4ref_cache *c, const uint16_t *q16, int32_t L, int32_t E,
                             int32_t slot, int g, const int32_t *row, float scale_log2,
                             int32_t pv_exact, double *out, double *lse, int8_t *dqc, int32_t *dqs,
                             int32_t *dqk, uint8_t *dpc, int32_t *dpv) {
  float qr[HD];
  for (int i = 0; i < HD; i++) qr[i] = kv4ref_bf16_to_f32(q16[i]);
  fwht128(qr); /* same rotation as the keys: scores are preserved */
  int8_t qc[HD];
  float s_q;
  int32_t qsum;
  quant_query(qr, qc, &s_q, &qsum);
  const float c_q = s_q * scale_log2;
  if (dqc) memcpy(dqc, qc, HD);
  if (dqs) *dqs = qsum;
  int32_t main_end = E - c->window; /* M = [s, main_end) */
  if (main_end > L) main_end = L;
  const int j0 = c->sink / PAGE;                                          /* first main page */
  const int j1 = main_end > c->sink ? (main_end - 1) / PAGE : j0 - 1;   /* last main page */
  const int ntiles = j1 - j0 + 1;
  partial_t *parts = (partial_t *)malloc(sizeof(partial_t) * (size_t)(ntiles + 1));
  protected_region(c, slot, g, L, E, qc, c_q, &parts[0], dqk);
  for (int j = j0; j <= j1; j++) {
    const uint8_t *blk = block_at(c, row[j], g);
    int t_end = main_end - PAGE * j;
    if (t_end > PAGE) t_end = PAGE;
    main_tile(blk, t_end, qc, qsum, c_q, pv_exact, &parts[1 + j - j0], dqk ? dqk + PAGE * j : NULL,
              dpc ? dpc + PAGE * j : NULL, dpv ? dpv + (size_t)j * HD : NULL);
  }
  merge(parts, ntiles + 1, out, lse);
  free(parts);
}

int kv4ref_decode(const kv4ref_cache *c, const uint16_t *q, const int32_t *ctx_len,
                  const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B,
                  int32_t Hq, float softmax_scale, int32_t pv_exact, double *out, double *lse,
                  const kv4ref_debug *dbg, int32_t nthreads) {
  exp2_init();
  const int Hkv = c->num_kv_heads;
  if (Hkv <= 0 || Hq % Hkv != 0 || !budget_ok(c)) return -1;
  const int G = Hq / Hkv; /* q-head h reads kv-head h / G */
  const float scale_log2 = kv4ref_scale_log2(softmax_scale);
  int bad = 0;

#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int bh = 0; bh < B * Hq; bh++) {
    const int b = bh / Hq, h = bh % Hq, g = h / G;
    const int32_t L = ctx_len[b];
    if (L < 1 || (L + PAGE - 1) / PAGE > pt_stride) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    decode_one_query(c, q + (size_t)bh * HD, L, L, slot ? slot[b] : b, g,
                     page_table + (size_t)b * pt_stride, scale_log2, pv_exact, out + (size_t)bh * HD,
                     lse + bh, (dbg && dbg->qcodes) ? dbg->qcodes + (size_t)bh * HD : NULL,
                     (dbg && dbg->qsum) ? dbg->qsum + bh : NULL,
                     (dbg && dbg->qk) ? dbg->qk + (size_t)bh * dbg->max_ctx : NULL,
                     (dbg && dbg->pcode) ? dbg->pcode + (size_t)bh * dbg->max_ctx : NULL,
                     (dbg && dbg->pv) ? dbg->pv + (size_t)bh * dbg->max_pages * HD : NULL);
  }
  return bad ? -2 : 0;
}

/* Re-prefill (chunked-prefill) attention over the cache: sequence s's chunk of
 * n_s = cu[s+1] - cu[s] query tokens at positions start[s] .. start[s]+n_s-1,
 * whose K/V the cache already holds (the cache ends at E = start[s] + n_s);
 * query token i attends [0, start[s] + i] with the protected set of that cache
 * state.  q, out: [T][Hq][128] with T = cu[nseq]; dbg indexed by token. */
int kv4ref_prefill_attention(const kv4ref_cache *c, const uint16_t *q, const int32_t *cu_seqlens,
                             const int32_t *start_pos, const int32_t *slot,
                             const int32_t *page_table, int32_t pt_stride, int32_t nseq, int32_t Hq,
                             float softmax_scale, int32_t pv_exact, double *out, double *lse,
                             const kv4ref_debug *dbg, int32_t nthreads) {
  exp2_init();
  const int Hkv = c->num_kv_heads;
  if (Hkv <= 0 || Hq % Hkv != 0 || !budget_ok(c)) return -1;
  const int G = Hq / Hkv;
  const float scale_log2 = kv4ref_scale_log2(softmax_scale);
  const int32_t T = cu_seqlens[nseq];
  int bad = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t th = 0; th < (int64_t)T * Hq; th++) {
    const int32_t t = (int32_t)(th / Hq), h = (int32_t)(th % Hq), g = h / G;
    int sq = 0;
    while (cu_seqlens[sq + 1] <= t) sq++;
    const int32_t L = start_pos[sq] + (t - cu_seqlens[sq]) + 1;
    const int32_t E = start_pos[sq] + (cu_seqlens[sq + 1] - cu_seqlens[sq]);
    if ((E + PAGE - 1) / PAGE > pt_stride) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    decode_one_query(c, q + (size_t)th * HD, L, E, slot ? slot[sq] : sq, g,
                     page_table + (size_t)sq * pt_stride, scale_log2, pv_exact, out + (size_t)th * HD,
                     lse + th, (dbg && dbg->qcodes) ? dbg->qcodes + (size_t)th * HD : NULL,
                     (dbg && dbg->qsum) ? dbg->qsum + th : NULL,
                     (dbg && dbg->qk) ? dbg->qk + (size_t)th * dbg->max_ctx : NULL,
                     (dbg && dbg->pcode) ? dbg->pcode + (size_t)th * dbg->max_ctx : NULL,
                     (dbg && dbg->pv) ? dbg->pv + (size_t)th * dbg->max_pages * HD : NULL);
  }
  return bad ? -2 : 0;
}

/* The same attention for a chosen list of (token, q-head) pairs only,
 * th[i] = token * Hq + head; out [n][128], lse [n].  For checking samples of
 * chunks too long to attend in full on the CPU. */
int kv4ref_prefill_attention_sampled(const kv4ref_cache *c, const uint16_t *q, const int32_t *cu_seqlens,
                                     const int32_t *start_pos, const int32_t *slot,
                                     const int32_t *page_table, int32_t pt_stride, int32_t nseq,
                                     int32_t Hq, float softmax_scale, int32_t n, const int64_t *th,
                                     double *out, double *lse, int32_t nthreads) {
  exp2_init();
  const int Hkv = c->num_kv_heads;
  if (Hkv <= 0 || Hq % Hkv != 0 || !budget_ok(c)) return -1;
  const int G = Hq / Hkv;
  const float scale_log2 = kv4ref_scale_log2(softmax_scale);
  const int64_t T = cu_seqlens[nseq];
  int bad = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int32_t i = 0; i < n; i++) {
    if (th[i] < 0 || th[i] >= T * Hq) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    const int32_t t = (int32_t)(th[i] / Hq), h = (int32_t)(th[i] % Hq), g = h / G;
    int sq = 0;
    while (cu_seqlens[sq + 1] <= t) sq++;
    const int32_t L = start_pos[sq] + (t - cu_seqlens[sq]) + 1;
    const int32_t E = start_pos[sq] + (cu_seqlens[sq + 1] - cu_seqlens[sq]);
    if ((E + PAGE - 1) / PAGE > pt_stride) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    decode_one_query(c, q + (size_t)th[i] * HD, L, E, slot ? slot[sq] : sq, g,
                     page_table + (size_t)sq * pt_stride, scale_log2, 0, out + (size_t)i * HD, lse + i,
                     NULL, NULL, NULL, NULL, NULL);
  }
  return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* KV8 everywhere: the INT8 comparison variant of the quantization-target     */
/* comparisons (KV4-RL pages, quantization-target comparison, figure 3).     */
/* Every position is stored as the side rows store the protected positions  */
/* (keys rotated, symmetric INT8 per 128-dim vector with an FP16 scale) and  */
/* attended with the protected path's arithmetic.  Pool layout per (page,    */
/* kv-head), 4160 B: K codes [16 positions][128] | V codes [128 channels][16 */
/* positions] | s_k FP16 [16] | s_v FP16 [16].                               */
/* ------------------------------------------------------------------------ */

enum { KV8_BLOCK = 4160, KV8_OFF_V = 2048, KV8_OFF_SK = 4096, KV8_OFF_SV = 4128 };

static uint8_t *kv8_block(const kv8ref_cache *c, int32_t phys, int g) {
  assert(phys >= 0 && phys < c->num_pages);
  return c->pages + ((size_t)phys * (size_t)c->num_kv_heads + (size_t)g) * KV8_BLOCK;
}

static void kv8_append_one(const kv8ref_cache *c, int g, const uint16_t *k16, const uint16_t *v16,
                           int32_t pos, const int32_t *table_row) {
  float k[HD], v[HD];
  for (int i = 0; i < HD; i++) {
    k[i] = kv4ref_bf16_to_f32(k16[i]);
    v[i] = kv4ref_bf16_to_f32(v16[i]);
  }
  fwht128(k);
  int8_t kc[HD], vc[HD];
  uint16_t ks, vs;
  quant_int8(k, kc, &ks);
  quant_int8(v, vc, &vs);
  uint8_t *blk = kv8_block(c, table_row[pos / PAGE], g);
  const int t = pos % PAGE;
  memcpy(blk + (size_t)t * HD, kc, HD);
  for (int j = 0; j < HD; j++) blk[KV8_OFF_V + j * PAGE + t] = (uint8_t)vc[j];
  memcpy(blk + KV8_OFF_SK + 2 * t, &ks, 2);
  memcpy(blk + KV8_OFF_SV + 2 * t, &vs, 2);
}

int kv8ref_append(const kv8ref_cache *c, const uint16_t *k, const uint16_t *v, const int32_t *pos,
                  const int32_t *page_table, int32_t pt_stride, int32_t B) {
  const int H = c->num_kv_heads;
  for (int b = 0; b < B; b++)
    for (int g = 0; g < H; g++) {
      size_t off = ((size_t)b * H + g) * HD;
      kv8_append_one(c, g, k + off, v + off, pos[b], page_table + (size_t)b * pt_stride);
    }
  return 0;
}

int kv8ref_prefill(const kv8ref_cache *c, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *page_table,
                   int32_t pt_stride, int32_t nseq, int32_t nthreads) {
  const int H = c->num_kv_heads;
  (void)nthreads;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int sq = 0; sq < nseq; sq++)
    for (int32_t i = 0; i < cu_seqlens[sq + 1] - cu_seqlens[sq]; i++) {
      size_t tok = (size_t)cu_seqlens[sq] + (size_t)i;
      for (int g = 0; g < H; g++) {
        size_t off = (tok * H + g) * HD;
        kv8_append_one(c, g, k + off, v + off, start_pos[sq] + i, page_table + (size_t)sq * pt_stride);
      }
    }
  return 0;
}

int kv8ref_decode(const kv8ref_cache *c, const uint16_t *q, const int32_t *ctx_len,
                  const int32_t *page_table, int32_t pt_stride, int32_t B, int32_t Hq,
                  float softmax_scale, double *out, double *lse, const kv4ref_debug *dbg,
                  int32_t nthreads) {
  exp2_init();
  const int Hkv = c->num_kv_heads;
  if (Hkv <= 0 || Hq % Hkv != 0) return -1;
  const int G = Hq / Hkv;
  const float scale_log2 = kv4ref_scale_log2(softmax_scale);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int bh = 0; bh < B * Hq; bh++) {
    const int b = bh / Hq, h = bh % Hq, g = h / G;
    const int32_t L = ctx_len[b];
    if (L < 1 || (L + PAGE - 1) / PAGE > pt_stride) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    float qr[HD];
    for (int i = 0; i < HD; i++) qr[i] = kv4ref_bf16_to_f32(q[(size_t)bh * HD + i]);
    fwht128(qr);
    int8_t qc[HD];
    float s_q;
    int32_t qsum;
    quant_query(qr, qc, &s_q, &qsum);
    if (dbg && dbg->qcodes) memcpy(dbg->qcodes + (size_t)bh * HD, qc, HD);
    if (dbg && dbg->qsum) dbg->qsum[bh] = qsum;
    int32_t *dqk = (dbg && dbg->qk) ? dbg->qk + (size_t)bh * dbg->max_ctx : NULL;
    int8_row_t *rows = (int8_row_t *)malloc(sizeof(int8_row_t) * (size_t)L);
    int8_t *vt = (int8_t *)malloc((size_t)L * HD); /* V codes of each position, channel order */
    const int32_t *trow = page_table + (size_t)b * pt_stride;
    for (int32_t p = 0; p < L; p++) {
      const uint8_t *blk = kv8_block(c, trow[p / PAGE], g);
      const int t = p % PAGE;
      for (int j = 0; j < HD; j++) vt[(size_t)p * HD + j] = (int8_t)blk[KV8_OFF_V + j * PAGE + t];
      rows[p].pos = p;
      rows[p].k8 = (const int8_t *)blk + (size_t)t * HD;
      rows[p].v8 = vt + (size_t)p * HD;
      memcpy(&rows[p].sk, blk + KV8_OFF_SK + 2 * t, 2);
      memcpy(&rows[p].sv, blk + KV8_OFF_SV + 2 * t, 2);
    }
    partial_t part;
    int8_region(rows, L, qc, s_q * scale_log2, &part, dqk);
    merge(&part, 1, out + (size_t)bh * HD, lse + bh);
    free(vt);
    free(rows);
  }
  return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 variant (KV4-RL pages, comparison of 4-bit formats, appendix D.4):  */
/* the main region stored in OCP MXFP4 instead of INT4 group-affine; the     */
/* rotation, the INT8 side buffer, the protected path and the merge are as   */
/* above.  Block per (page, kv-head), 2176 B: K codes [16][64] (E2M1, channel */
/* 2i low nibble of byte i) | V codes [128][8] (channel-major, position 2k   */
/* low nibble of byte k) | K scales E8M0 [16 positions][4 blocks] | V scales */
/* E8M0 [16][4]; block b = channels 32b .. 32b+31.                           */
/* ------------------------------------------------------------------------ */

enum { MX_OFF_V = 1024, MX_OFF_KS = 2048, MX_OFF_VS = 2112 };

/* E2M1 value of a 4-bit code: sign, 2 exponent bits (bias 1), 1 mantissa bit. */
static double e2m1_value(int code) {
  const int e = (code >> 1) & 3, m = code & 1;
  const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
  return (code & 8) ? -mag : mag;
}

/* Nearest E2M1 code of y (ties to the even mantissa), saturating at +-6; the
 * sign bit follows y's sign (so -0.2 gives the code of -0). */
static int e2m1_code(double y) {
  const double a = fabs(y);
  int best = 0;
  for (int c = 1; c < 8; c++) {
    const double d = fabs(e2m1_value(c) - a), db = fabs(e2m1_value(best) - a);
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  if (a > 6.0) best = 7;
  return best | (signbit(y) ? 8 : 0);
}

/* OCP MX block quantizer: E = floor(log2(amax)) - 2 (2 = largest E2M1
 * exponent), clamped to [-127, 127], E = -127 for an all-zero block; codes =
 * E2M1 of x / 2^E.  Returns the E8M0 byte E + 127. */
static uint8_t mx_block(const float *x, uint8_t *codes /* 32 */) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
  int E = -127;
  if (amax > 0.0f) {
    int ex;
    frexpf(amax, &ex); /* amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    E = ex - 1 - 2;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
  }
  for (int i = 0; i < 32; i++) codes[i] = (uint8_t)e2m1_code(ldexp((double)x[i], -E));
  return (uint8_t)(E + 127);
}

static void mx_append_one(const kv4ref_cache *c, int g, const uint16_t *k16, const uint16_t *v16,
                          int32_t pos, int32_t slot, const int32_t *table_row) {
  float k[HD], v[HD];
  for (int i = 0; i < HD; i++) {
    k[i] = kv4ref_bf16_to_f32(k16[i]);
    v[i] = kv4ref_bf16_to_f32(v16[i]);
  }
  fwht128(k);
  uint8_t *blk = block_at(c, table_row[pos / PAGE], g);
  const int t = pos % PAGE;
  for (int b = 0; b < 4; b++) {
    uint8_t kc[32], vc[32];
    blk[MX_OFF_KS + 4 * t + b] = mx_block(k + 32 * b, kc);
    blk[MX_OFF_VS + 4 * t + b] = mx_block(v + 32 * b, vc);
    for (int i = 0; i < 16; i++) blk[64 * t + 16 * b + i] = (uint8_t)(kc[2 * i] | (kc[2 * i + 1] << 4));
    for (int i = 0; i < 32; i++) {
      uint8_t *byte = blk + MX_OFF_V + 8 * (32 * b + i) + t / 2;
      *byte = (t & 1) ? (uint8_t)((*byte & 0x0F) | (vc[i] << 4)) : (uint8_t)((*byte & 0xF0) | vc[i]);
    }
  }
  int row = side_row(c, pos);
  if (row < 0) return;
  quant_int8(k, side_code_at(c, slot, g, row, 0), side_scale_at(c, slot, g, row, 0));
  quant_int8(v, side_code_at(c, slot, g, row, 1), side_scale_at(c, slot, g, row, 1));
}

int mxref_append(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v, const int32_t *pos,
                 const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B) {
  const int H = c->num_kv_heads;
  if (!budget_ok(c)) return -1;
  for (int b = 0; b < B; b++)
    for (int g = 0; g < H; g++) {
      size_t off = ((size_t)b * H + g) * HD;
      mx_append_one(c, g, k + off, v + off, pos[b], slot ? slot[b] : b,
                    page_table + (size_t)b * pt_stride);
    }
  return 0;
}

int mxref_prefill(const kv4ref_cache *c, const uint16_t *k, const uint16_t *v,
                  const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *slot,
                  const int32_t *page_table, int32_t pt_stride, int32_t nseq, int32_t nthreads) {
  const int H = c->num_kv_heads;
  (void)nthreads;
  if (!budget_ok(c)) return -1;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int sq = 0; sq < nseq; sq++)
    for (int32_t i = 0; i < cu_seqlens[sq + 1] - cu_seqlens[sq]; i++) {
      size_t tok = (size_t)cu_seqlens[sq] + (size_t)i;
      for (int g = 0; g < H; g++) {
        size_t off = (tok * H + g) * HD;
        mx_append_one(c, g, k + off, v + off, start_pos[sq] + i, slot ? slot[sq] : sq,
                      page_table + (size_t)sq * pt_stride);
      }
    }
  return 0;
}

/* Dequantized MXFP4 entry t of a block (exact). */
static void mx_unpack(const uint8_t *blk, int t, double k[HD], double v[HD]) {
  for (int j = 0; j < HD; j++) {
    const int kc = (blk[64 * t + j / 2] >> (4 * (j & 1))) & 15;
    const int vcd = (blk[MX_OFF_V + 8 * j + t / 2] >> (4 * (t & 1))) & 15;
    k[j] = ldexp(e2m1_value(kc), (int)blk[MX_OFF_KS + 4 * t + j / 32] - 127);
    v[j] = ldexp(e2m1_value(vcd), (int)blk[MX_OFF_VS + 4 * t + j / 32] - 127);
  }
}

/* Main region of the MXFP4 variant, one partial: z = (bf16(q_rot) . k^) *
 * scale_log2 (the dot exact, rounded once to FP32), e = exp2s(z - z_max) in
 * FP32, A = sum e v^ with the exactly dequantized values. */
static void mx_main(const kv4ref_cache *c, const int32_t *trow, int g, int32_t m0, int32_t m1,
                    const float qb[HD], float scale_log2, partial_t *out) {
  out->Z = -INFINITY;
  out->l = 0.0;
  for (int j = 0; j < HD; j++) out->A[j] = 0.0;
  const int n = m1 - m0;
  if (n <= 0) return;
  float *z = (float *)malloc(sizeof(float) * (size_t)n);
  double *vals = (double *)malloc(sizeof(double) * (size_t)n * HD);
  float zmax = -INFINITY;
  for (int i = 0; i < n; i++) {
    const int p = m0 + i;
    double kk[HD];
    mx_unpack(block_at(c, trow[p / PAGE], g), p % PAGE, kk, vals + (size_t)i * HD);
    double d = 0.0;
    for (int j = 0; j < HD; j++) d += (double)qb[j] * kk[j]; /* exact: few significant bits */
    z[i] = (float)d * scale_log2;
    if (z[i] > zmax) zmax = z[i];
  }
  out->Z = zmax;
  for (int i = 0; i < n; i++) {
    const float e = exp2s(z[i] - zmax);
    out->l += (double)e;
    for (int j = 0; j < HD; j++) out->A[j] += (double)e * vals[(size_t)i * HD + j];
  }
  free(vals);
  free(z);
}

int mxref_decode(const kv4ref_cache *c, const uint16_t *q, const int32_t *ctx_len,
                 const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B,
                 int32_t Hq, float softmax_scale, double *out, double *lse, int32_t nthreads) {
  exp2_init();
  const int Hkv = c->num_kv_heads;
  if (Hkv <= 0 || Hq % Hkv != 0 || !budget_ok(c)) return -1;
  const int G = Hq / Hkv;
  const float scale_log2 = kv4ref_scale_log2(softmax_scale);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int bh = 0; bh < B * Hq; bh++) {
    const int b = bh / Hq, h = bh % Hq, g = h / G;
    const int32_t L = ctx_len[b];
    if (L < 1 || (L + PAGE - 1) / PAGE > pt_stride) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    float qr[HD];
    for (int i = 0; i < HD; i++) qr[i] = kv4ref_bf16_to_f32(q[(size_t)bh * HD + i]);
    fwht128(qr);
    int8_t qc[HD];
    float s_q, qb[HD];
    int32_t qsum;
    quant_query(qr, qc, &s_q, &qsum);
    for (int i = 0; i < HD; i++) qb[i] = kv4ref_bf16_to_f32(kv4ref_f32_to_bf16(qr[i]));
    partial_t parts[2];
    protected_region(c, slot ? slot[b] : b, g, L, L, qc, s_q * scale_log2, &parts[0], NULL);
    const int32_t main_end = L - c->window;
    mx_main(c, page_table + (size_t)b * pt_stride, g, c->sink, main_end > c->sink ? main_end : c->sink,
            qb, scale_log2, &parts[1]);
    merge(parts, 2, out + (size_t)bh * HD, lse + bh);
  }
  return bad ? -2 : 0;
}
