/*
 * kv4.h -- C ABI of the KV4-RL hybrid decode-attention library (MI355X, gfx950).
 *
 * The operations follow the KV4-RL pages (paper.rainbus.top summary,
 * "方法步骤详情" steps 2-4 and "核心方法"; onedev.kr summary, "전제와 한계"):
 *   - every cached position of K and V is group-affine INT4 (one group per
 *     128-dim token-head vector, x^ = delta*c + m, FP16 delta and m computed on
 *     line), 4.25 bits per element; keys are Hadamard-rotated after RoPE;
 *   - the first s (sink) and last w (recent) positions also have an INT8 copy
 *     in a fixed-capacity side buffer (s = 16, w = 128 in the pages' main
 *     configuration; other budgets, s = w = 0 included, are the allocation
 *     comparisons of their figures 3 and 4(b)); leaving the window rewrites
 *     nothing;
 *   - one decode step quantizes the rotated query to INT8 once, runs integer
 *     QK and integer PV over the INT4 main region and INT8 QK / BF16 V / FP32 PV
 *     over the protected region, and merges the two exactly.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (HIP global memory) unless a
 *     comment says otherwise; descriptors and debug structs live on the host.
 *   - The caller owns all memory.  The library never allocates, frees or
 *     synchronizes, keeps no state between calls (apart from the fixed scratch
 *     array of kv4_append_decode_attention_noalloc), and enqueues its work on the
 *     given HIP stream (`hipStream_t` passed as void*; NULL = default stream).
 *     Calls are stream-ordered: an append followed by a decode on the same
 *     stream sees the appended token.
 *   - Return value: KV4_OK (0) or a negative KV4_ERR_* code; no exception
 *     crosses the ABI.  Host-checkable argument errors are reported before
 *     anything is enqueued.  Device-side contracts (1 <= ctx_len <= max_ctx,
 *     valid page ids, slot < max_slots, positions inside the page table) are
 *     not checked on the device.
 *   - BF16/FP16 tensors are 16-bit IEEE patterns; all device pointers must be
 *     16-byte aligned.
 */
#ifndef KV4_H
#define KV4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV4_ABI_VERSION 1

enum {
  KV4_OK = 0,
  KV4_ERR_NULLPTR = -1,     /* a required pointer is NULL */
  KV4_ERR_UNSUPPORTED = -2, /* head_dim != 128, page_size != 16, sink < 0,
                               window < 0, sink % 16 != 0, sink + window > 144,
                               Hq % Hkv != 0 (any G = Hq / Hkv >= 1 is taken:
                               the kernels work on groups of up to 4 query
                               heads of one kv-head; only the BF16 comparator
                               needs G = 4), or abi_version mismatch */
  KV4_ERR_SHAPE = -3,       /* a size is out of range (B <= 0, max_ctx > pt_stride*16,
                               B * num_kv_heads * ceil(G/4) * (max_ctx/16 + 1) > INT32_MAX, ...) */
  KV4_ERR_WORKSPACE = -4,   /* workspace missing or smaller than kv4_decode_workspace_bytes
                               (no-allocation entry point: more than its fixed scratch) */
  KV4_ERR_HIP = -5          /* a HIP call failed; kv4_strerror gives the HIP message */
};

/* One layer's cache (host-side descriptor of caller-owned device memory).
 *   pages        uint8 [num_pages][num_kv_heads][2176]: one block per
 *                (physical page, kv-head) = K codes 1024 B (position t at bytes
 *                64t..64t+63, channel 2i in the low nibble of byte i, 2i+1 in
 *                the high nibble) | V codes 1024 B (channel j at bytes
 *                8j..8j+7, position 2k in the low nibble of byte k, 2k+1 in
 *                the high nibble) | 16 x {delta, m} FP16 for K | same for V.
 *   side_codes   int8  [max_slots][num_kv_heads][144][2][128]: INT8 copies,
 *                K (rotated) then V, of sink positions (row p for p < s) and
 *                recent positions (row s + p mod w); rows past s + w unused.
 *   side_scales  fp16  [max_slots][num_kv_heads][144][2]: their scales. */
typedef struct kv4_cache_desc {
  int32_t abi_version; /* KV4_ABI_VERSION */
  int32_t num_pages;
  int32_t page_size;   /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;    /* must be 128 */
  int32_t sink;        /* s: protected leading positions, a multiple of 16 (16) */
  int32_t window;      /* w: protected recent positions (128); s + w <= 144.
                          s = w = 0 is unprotected KV4.  A cache must be
                          written and read with the same s and w. */
  int32_t max_slots;
  void *pages;
  void *side_codes;
  void *side_scales;
} kv4_cache_desc;

/* Quantize-on-append of one token per sequence (steps 2-3 of the pages).
 *   k, v        bf16 [B][num_kv_heads][128], post-RoPE keys and values
 *   pos         int32 [B], position of the token in its sequence
 *   slot        int32 [B], side-buffer slot of each sequence (NULL = b)
 *   page_table  int32 [B][pt_stride], logical page -> physical page; entry
 *               pos/16 must name a page owned by sequence b
 * Writes the INT4 codes and FP16 delta/m of K (rotated) and V into slot pos%16
 * of page page_table[b][pos/16], and the INT8 side row of pos (sinks for
 * pos < s, the recent ring otherwise; none when pos >= s and w = 0).  The INT4 entry of the position
 * leaving the window is not touched.  Two entries of one call must not write
 * the same position. */
int kv4_append(const kv4_cache_desc *cache, const void *k, const void *v, const int32_t *pos,
               const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B,
               void *stream);

/* Bulk re-prefill of carried prefixes (step 1 of the pages): quantizes T
 * tokens exactly as T appends at positions start_pos[s] .. start_pos[s]+n_s-1
 * would, leaving byte-identical pages and side rows.
 *   k, v        bf16 [T][num_kv_heads][128], sequences back to back
 *   cu_seqlens  int32 [nseq+1], token offsets (cu_seqlens[0] = 0)
 *   start_pos   int32 [nseq], first position of each sequence's tokens
 *   slot        int32 [nseq] (NULL = s);  page_table int32 [nseq][pt_stride]
 *   max_seqlen  host upper bound of max_s (start_pos[s] % 16 + n_s), sizes the grid */
int kv4_prefill_quantize(const kv4_cache_desc *cache, const void *k, const void *v,
                         const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *slot,
                         const int32_t *page_table, int32_t pt_stride, int32_t nseq,
                         int32_t max_seqlen, void *stream);

/* Bytes of device workspace kv4_decode_attention needs for B sequences and
 * Hq query heads on the current device (0 on bad arguments). */
size_t kv4_decode_workspace_bytes(const kv4_cache_desc *cache, int32_t B, int32_t Hq,
                                  int32_t max_ctx);

/* One decode step of hybrid attention (step 4 of the pages).
 *   q          bf16 [B][Hq][128], post-RoPE queries; q-head h reads kv-head h/(Hq/Hkv)
 *   ctx_len    int32 [B], context length INCLUDING this step's token: attends [0, ctx_len)
 *   slot, page_table, pt_stride as for kv4_append
 *   max_ctx    host upper bound of ctx_len (<= pt_stride * 16)
 *   softmax_scale  logit scale (typically 1/sqrt(128))
 *   out        fp32 [B][Hq][128], attention output
 *   lse        fp32 [B][Hq], natural-log normaliser of the softmax
 *   workspace  device scratch of at least kv4_decode_workspace_bytes bytes
 * Positions [s, ctx_len-w) are read from the INT4 pages; [0, min(s, ctx_len))
 * and [max(s, ctx_len-w), ctx_len) from the INT8 side rows. */
int kv4_decode_attention(const kv4_cache_desc *cache, const void *q, const int32_t *ctx_len,
                         const int32_t *slot, const int32_t *page_table, int32_t pt_stride,
                         int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale, float *out,
                         float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* One whole decode step in one launch: kv4_append(k, v, pos) followed by
 * kv4_decode_attention, with identical results.  Requires pos[b] = ctx_len[b]
 * - 1 (this step's token; not checked on the device).  When w > 0 the token
 * lies in its sequence's recent window, so the protected-region workgroup of
 * (b, kv-head) quantizes and writes it (page entry and side row) before it
 * attends, and no other work of the step reads it; with w = 0 the append runs
 * as its own launch first.  Arguments as for the two calls. */
int kv4_append_decode_attention(const kv4_cache_desc *cache, const void *k, const void *v,
                                const int32_t *pos, const void *q, const int32_t *ctx_len,
                                const int32_t *slot, const int32_t *page_table, int32_t pt_stride,
                                int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale,
                                float *out, float *lse, void *workspace, size_t workspace_bytes,
                                void *stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * kv4_append_decode_attention with the workspace taken from a fixed scratch
 * array inside the library instead of a caller buffer; the same kernels, the
 * same results bit for bit.  No allocation or free of any kind happens in the
 * call.  The array holds KV4_NOALLOC_SCRATCH_BYTES on every GPU the library
 * runs on, from the first call on that GPU until the process ends; a call
 * whose kv4_decode_workspace_bytes exceeds it returns KV4_ERR_WORKSPACE before
 * anything is enqueued (32 MiB covers B = 512 sequences at Hq/Hkv = 32/8 on a
 * 256-CU device).  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (different streams, or host threads racing on one
 * stream) race on it: serialize them.  Nothing in the array has to start at
 * zero, so what an earlier call left there does not matter.  Arguments,
 * layouts and other errors as for kv4_append_decode_attention. */
#define KV4_NOALLOC_SCRATCH_BYTES (32u << 20)
int kv4_append_decode_attention_noalloc(const kv4_cache_desc *cache, const void *k, const void *v,
                                        const int32_t *pos, const void *q, const int32_t *ctx_len,
                                        const int32_t *slot, const int32_t *page_table,
                                        int32_t pt_stride, int32_t B, int32_t Hq, int32_t max_ctx,
                                        float softmax_scale, float *out, float *lse, void *stream);

/* Integer intermediates of a decode step, for bit-exact checking (device
 * pointers; any may be NULL).  Same layouts as the arguments of
 * kv4_decode_attention plus:
 *   qcodes  int8  [B][Hq][128]   INT8 codes of the rotated query
 *   qsum    int32 [B][Hq]        their sum
 *   qk      int32 [B][Hq][max_ctx]  integer Q.K of each attended position
 *   pcode   uint8 [B][Hq][max_ctx]  P-operand code of each main position
 *   pv      int32 [B][Hq][max_pages][128]  integer P.V accumulators of the
 *                                 main tile on logical page j (j >= s/16) */
typedef struct kv4_decode_debug {
  int8_t *qcodes;
  int32_t *qsum;
  int32_t *qk;
  uint8_t *pcode;
  int32_t *pv;
  int32_t max_ctx;
  int32_t max_pages;
} kv4_decode_debug;

/* kv4_decode_attention running the same kernels instantiated with extra
 * stores of the integer intermediates into *dbg (a host struct). */
int kv4_decode_attention_debug(const kv4_cache_desc *cache, const void *q,
                               const int32_t *ctx_len, const int32_t *slot,
                               const int32_t *page_table, int32_t pt_stride, int32_t B,
                               int32_t Hq, int32_t max_ctx, float softmax_scale, float *out,
                               float *lse, void *workspace, size_t workspace_bytes,
                               const kv4_decode_debug *dbg, void *stream);

/* ---- re-prefill (chunked-prefill) attention ----------------------------------
 * The attention half of carried-prefix re-prefill (step 1 of the pages), over
 * the KV4-RL cache after kv4_prefill_quantize wrote the chunk: sequence s has
 * n_s = cu_seqlens[s+1] - cu_seqlens[s] query tokens at positions start_pos[s]
 * .. start_pos[s] + n_s - 1, and its cache now ends at E_s = start_pos[s] + n_s.
 * Token i attends [0, start_pos[s] + i]: the sinks and the positions of the
 * cache's recent window [max(s, E_s - w), E_s) it can see from the INT8 side
 * rows, the rest of [s, min(p + 1, E_s - w)) from the INT4 pages, with the
 * rules of kv4_decode_attention (a one-token chunk is a decode step).
 *   q          bf16 [total_q][Hq][128] (total_q = cu_seqlens[nseq])
 *   slot, page_table, pt_stride: per sequence, as for kv4_prefill_quantize
 *   max_ctx    host upper bound of E_s
 *   out, lse   fp32 [total_q][Hq][128], [total_q][Hq]
 * One workgroup per (block of 8 consecutive tokens of a chunk, group of up to 4
 * query heads of one kv-head) covers
 * the block's protected rows and main tiles, so every INT4 tile and side row
 * is read once per 8 tokens; the integer intermediates (query codes, QK, P
 * codes, PV accumulators) are those of the decode step, and out / lse equal it
 * up to the FP32 order of the exact region and tile merges.  The workspace
 * holds (total_q + 1) int32 block bases; nseq must not exceed total_q
 * (KV4_ERR_HIP otherwise). */
size_t kv4_prefill_attention_workspace_bytes(const kv4_cache_desc *cache, int32_t total_q,
                                             int32_t Hq, int32_t max_ctx);
int kv4_prefill_attention(const kv4_cache_desc *cache, const void *q, const int32_t *cu_seqlens,
                          const int32_t *start_pos, const int32_t *slot, const int32_t *page_table,
                          int32_t pt_stride, int32_t nseq, int32_t total_q, int32_t Hq,
                          int32_t max_ctx, float softmax_scale, float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream);
/* With the debug stores of kv4_decode_attention_debug, indexed by token. */
int kv4_prefill_attention_debug(const kv4_cache_desc *cache, const void *q,
                                const int32_t *cu_seqlens, const int32_t *start_pos,
                                const int32_t *slot, const int32_t *page_table, int32_t pt_stride,
                                int32_t nseq, int32_t total_q, int32_t Hq, int32_t max_ctx,
                                float softmax_scale, float *out, float *lse, void *workspace,
                                size_t workspace_bytes, const kv4_decode_debug *dbg, void *stream);

/* Static message for a status code (for KV4_ERR_HIP: the last HIP error seen
 * by this thread). */
const char *kv4_strerror(int status);

/* ---- comparator, not part of the method: plain BF16 paged decode ----------
 * The baseline the pages compare against is ordinary BF16 paged attention.
 *   pages   bf16 [num_pages][Hkv][2][16][128]: per (page, kv-head) 16 K rows
 *           then 16 V rows, unrotated
 *   q, ctx_len, page_table, out, lse as for kv4_decode_attention; Hq/Hkv = 4
 *   (other group sizes: KV4_ERR_UNSUPPORTED) */
size_t kv4bench_bf16_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_ctx);
int kv4bench_bf16_paged_decode(const void *pages, int32_t num_pages, int32_t Hkv, const void *q,
                               const int32_t *ctx_len, const int32_t *page_table,
                               int32_t pt_stride, int32_t B, int32_t Hq, int32_t max_ctx,
                               float softmax_scale, float *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Benchmark hook: kv4_append_decode_attention (k, v, pos given) or
 * kv4_decode_attention (all three NULL) that also records two caller-created
 * HIP events (hipEvent_t passed as void*) on `stream`, immediately before and
 * after the main kernel, so the dominant kernel can be timed on the stream it
 * runs on.  Either event may be NULL. */
int kv4bench_decode_attention_timed(const kv4_cache_desc *cache, const void *k, const void *v,
                                    const int32_t *pos, const void *q, const int32_t *ctx_len,
                                    const int32_t *slot, const int32_t *page_table,
                                    int32_t pt_stride, int32_t B, int32_t Hq, int32_t max_ctx,
                                    float softmax_scale, float *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *ev_main_begin, void *ev_main_end,
                                    void *stream);

/* ---- variant: MXFP4 main region ----------------------------------------------
 * The 4-bit format comparison of the pages (KV4-RL, appendix D.4: NVFP4 and
 * MXFP4 against INT4 group-affine): the same cache descriptor, budget, side
 * buffer and protected path, with each page block (2176 B) holding the main
 * region in OCP MXFP4 instead: K codes [16 positions][64 B] (E2M1, channel 2i
 * in the low nibble of byte i, keys Hadamard-rotated) | V codes [128
 * channels][8 B] (position 2k low nibble of byte k) | K scales E8M0 [16][4] |
 * V scales E8M0 [16][4], one scale per 32-channel block: E = floor(log2 amax)
 * - 2 (clamped to [-127, 127], -127 for an all-zero block), code = E2M1 of
 * x / 2^E rounded to nearest even and saturated at 6.  The main region is
 * attended on the exactly dequantized values: logits from the BF16-rounded
 * rotated query, FP32 softmax weights, FP32 accumulation.  A cache must be
 * written and read by the same variant. */
int kv4mx_append(const kv4_cache_desc *cache, const void *k, const void *v, const int32_t *pos,
                 const int32_t *slot, const int32_t *page_table, int32_t pt_stride, int32_t B,
                 void *stream);
int kv4mx_prefill_quantize(const kv4_cache_desc *cache, const void *k, const void *v,
                           const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *slot,
                           const int32_t *page_table, int32_t pt_stride, int32_t nseq,
                           int32_t max_seqlen, void *stream);
/* Workspace as kv4_decode_workspace_bytes; arguments and errors as for
 * kv4_decode_attention. */
int kv4mx_decode_attention(const kv4_cache_desc *cache, const void *q, const int32_t *ctx_len,
                           const int32_t *slot, const int32_t *page_table, int32_t pt_stride,
                           int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale, float *out,
                           float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* ---- variant: KV8 everywhere ----------------------------------------------
 * The INT8 point of the pages' quantization-target comparison (KV4-RL,
 * quantization-target comparison, figure 3): every position is stored the way
 * the side buffer stores a protected position (key Hadamard-rotated after
 * RoPE, symmetric INT8 per 128-dim vector with an FP16 scale) and attended
 * with the protected path's arithmetic (the INT8 query against INT8 keys,
 * FP32 softmax weights, values dequantized to BF16, FP32 accumulation).
 *   pages  uint8 [num_pages][num_kv_heads][4160]: per (page, kv-head) K codes
 *          int8 [16 positions][128] | V codes int8 [128 channels][16
 *          positions] | s_k FP16 [16] | s_v FP16 [16]. */
typedef struct kv8_cache_desc {
  int32_t abi_version; /* KV4_ABI_VERSION */
  int32_t num_pages;
  int32_t page_size;   /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;    /* must be 128 */
  void *pages;
} kv8_cache_desc;

/* As kv4_append (no side buffer, no slot): writes the INT8 codes and scales
 * of position pos[b] into slot pos%16 of page page_table[b][pos/16]. */
int kv8_append(const kv8_cache_desc *cache, const void *k, const void *v, const int32_t *pos,
               const int32_t *page_table, int32_t pt_stride, int32_t B, void *stream);

/* As kv4_prefill_quantize: byte-identical to appends of the same tokens. */
int kv8_prefill_quantize(const kv8_cache_desc *cache, const void *k, const void *v,
                         const int32_t *cu_seqlens, const int32_t *start_pos,
                         const int32_t *page_table, int32_t pt_stride, int32_t nseq,
                         int32_t max_seqlen, void *stream);

/* Device workspace bytes of kv8_decode_attention (0 on bad arguments). */
size_t kv8_decode_workspace_bytes(const kv8_cache_desc *cache, int32_t B, int32_t Hq,
                                  int32_t max_ctx);

/* One decode step over positions [0, ctx_len) of every sequence; arguments,
 * layouts and errors as for kv4_decode_attention (no slot). */
int kv8_decode_attention(const kv8_cache_desc *cache, const void *q, const int32_t *ctx_len,
                         const int32_t *page_table, int32_t pt_stride, int32_t B, int32_t Hq,
                         int32_t max_ctx, float softmax_scale, float *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);

/* kv8_decode_attention with the debug stores: qcodes, qsum and qk of *dbg
 * (pcode and pv are not used). */
int kv8_decode_attention_debug(const kv8_cache_desc *cache, const void *q, const int32_t *ctx_len,
                               const int32_t *page_table, int32_t pt_stride, int32_t B,
                               int32_t Hq, int32_t max_ctx, float softmax_scale, float *out,
                               float *lse, void *workspace, size_t workspace_bytes,
                               const kv4_decode_debug *dbg, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KV4_H */
