// kv4_api.hip -- extern "C" entry points of libkv4 (declared in include/kv4.h):
// argument validation on the host, then stream-ordered kernel launches.  No
// allocation, no synchronization, no state kept between calls (apart from a
// per-device cache of the compute-unit count, a thread-local error text and
// the per-device address of the no-allocation entry point's fixed scratch).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kv4.h"
#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace {

thread_local char g_hip_error[256] = "no HIP error recorded";

int hip_fail(hipError_t e) {
  std::snprintf(g_hip_error, sizeof(g_hip_error), "HIP error %d: %s", static_cast<int>(e),
                hipGetErrorString(e));
  return KV4_ERR_HIP;
}

int check_cache(const kv4_cache_desc* c) {
  if (!c) return KV4_ERR_NULLPTR;
  if (c->abi_version != KV4_ABI_VERSION || c->page_size != 16 || c->head_dim != 128 ||
      c->sink < 0 || c->window < 0 || c->sink % 16 != 0 || c->sink + c->window > kv4::SIDE_ROWS)
    return KV4_ERR_UNSUPPORTED;
  if (c->num_pages <= 0 || c->num_kv_heads <= 0 || c->max_slots <= 0) return KV4_ERR_SHAPE;
  if (!c->pages || !c->side_codes || !c->side_scales) return KV4_ERR_NULLPTR;
  return KV4_OK;
}

kv4::CacheView view(const kv4_cache_desc* c) {
  return kv4::CacheView{static_cast<uint8_t*>(c->pages), static_cast<int8_t*>(c->side_codes),
                        static_cast<uint16_t*>(c->side_scales), c->num_pages, c->num_kv_heads,
                        c->max_slots, c->sink, c->window};
}

// softmax in base 2: logits carry softmax_scale * log2(e)
float scale_log2(float softmax_scale) {
  return static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634073599);
}

int check_decode(const kv4_cache_desc* c, const void* q, const int32_t* ctx,
                 const int32_t* page_table, int32_t pt_stride, int32_t B, int32_t Hq,
                 int32_t max_ctx, float* out, float* lse) {
  int rc = check_cache(c);
  if (rc != KV4_OK) return rc;
  if (!q || !ctx || !page_table || !out || !lse) return KV4_ERR_NULLPTR;
  if (Hq <= 0 || Hq % c->num_kv_heads != 0) return KV4_ERR_UNSUPPORTED;
  if (B <= 0 || pt_stride <= 0 || max_ctx <= 0 ||
      static_cast<int64_t>(max_ctx) > static_cast<int64_t>(pt_stride) * 16)
    return KV4_ERR_SHAPE;
  // main-region pages of all (sequence, query-head group) pairs are counted in int32
  if (static_cast<int64_t>(B) * kv4::query_head_groups(Hq, c->num_kv_heads) * (max_ctx / 16 + 1) > INT32_MAX)
    return KV4_ERR_SHAPE;
  return KV4_OK;
}

// ---- fixed scratch of the no-allocation entry point ------------------------
// The decode workspace of kv4_append_decode_attention_noalloc lives in this
// array: every GPU the library runs on holds its own copy for the life of the
// process.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in symbol); the device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[KV4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (nullptr and a recorded HIP
// error if the lookup fails).
void* scratch_for_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    hip_fail(hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace kv4 {
int main_region_waves() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    // 4 SIMDs per compute unit; at most 65536 waves (the split's 32-bit arithmetic)
    cached[dev] = std::min(cus, 4096) * 4 * KV4_MAIN_WAVES_PER_SIMD;
  }
  return cached[dev];
}
int kv8_region_waves() {
  return main_region_waves() / KV4_MAIN_WAVES_PER_SIMD * KV8_MAIN_WAVES_PER_SIMD;
}
}  // namespace kv4

extern "C" {

const char* kv4_strerror(int status) {
  switch (status) {
    case KV4_OK: return "success";
    case KV4_ERR_NULLPTR: return "a required pointer is NULL";
    case KV4_ERR_UNSUPPORTED:
      return "unsupported configuration (needs abi_version 1, page 16, head_dim 128, "
             "sink a multiple of 16, sink + window <= 144, Hq a multiple of Hkv; the BF16 "
             "comparator: Hq/Hkv = 4)";
    case KV4_ERR_SHAPE: return "a size argument is out of range";
    case KV4_ERR_WORKSPACE:
      return "workspace missing or smaller than kv4_decode_workspace_bytes (for "
             "kv4_append_decode_attention_noalloc: the batch needs more than its fixed "
             "KV4_NOALLOC_SCRATCH_BYTES of scratch)";
    case KV4_ERR_HIP: return g_hip_error;
    default: return "unknown status";
  }
}

int kv4_append(const kv4_cache_desc* cache, const void* k, const void* v, const int32_t* pos,
               const int32_t* slot, const int32_t* page_table, int32_t pt_stride, int32_t B,
               void* stream) {
  int rc = check_cache(cache);
  if (rc != KV4_OK) return rc;
  if (!k || !v || !pos || !page_table) return KV4_ERR_NULLPTR;
  if (B <= 0 || pt_stride <= 0 || B > 65535) return KV4_ERR_SHAPE;
  hipError_t e = kv4::launch_append(view(cache), static_cast<const uint16_t*>(k),
                                    static_cast<const uint16_t*>(v), pos, slot, page_table,
                                    pt_stride, B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv4_prefill_quantize(const kv4_cache_desc* cache, const void* k, const void* v,
                         const int32_t* cu_seqlens, const int32_t* start_pos, const int32_t* slot,
                         const int32_t* page_table, int32_t pt_stride, int32_t nseq,
                         int32_t max_seqlen, void* stream) {
  int rc = check_cache(cache);
  if (rc != KV4_OK) return rc;
  if (!k || !v || !cu_seqlens || !start_pos || !page_table) return KV4_ERR_NULLPTR;
  if (nseq <= 0 || nseq > 65535 || pt_stride <= 0 || max_seqlen <= 0) return KV4_ERR_SHAPE;
  hipError_t e = kv4::launch_prefill(view(cache), static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), cu_seqlens, start_pos, slot,
                                     page_table, pt_stride, nseq, max_seqlen,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

size_t kv4_decode_workspace_bytes(const kv4_cache_desc* cache, int32_t B, int32_t Hq,
                                  int32_t max_ctx) {
  if (check_cache(cache) != KV4_OK || B <= 0 || Hq <= 0 || Hq % cache->num_kv_heads != 0 || max_ctx <= 0)
    return 0;
  return kv4::decode_workspace_bytes(B, Hq, cache->num_kv_heads, kv4::main_region_waves());
}

static int decode_common(const kv4_cache_desc* cache, const void* q, const int32_t* ctx_len,
                         const int32_t* slot, const int32_t* page_table, int32_t pt_stride,
                         int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale, float* out,
                         float* lse, void* workspace, size_t workspace_bytes,
                         const kv4_decode_debug* dbg, void* stream, void* ev0 = nullptr,
                         void* ev1 = nullptr, bool mx = false, const void* k_new = nullptr,
                         const void* v_new = nullptr, const int32_t* pos_new = nullptr) {
  int rc = check_decode(cache, q, ctx_len, page_table, pt_stride, B, Hq, max_ctx, out, lse);
  if (rc != KV4_OK) return rc;
  if (B > 65535) return KV4_ERR_SHAPE;
  const int nw = kv4::main_region_waves();
  if (!workspace || workspace_bytes < kv4::decode_workspace_bytes(B, Hq, cache->num_kv_heads, nw))
    return KV4_ERR_WORKSPACE;
  kv4::DecodeDebug d{};
  if (dbg) {
    if (dbg->max_ctx < max_ctx || dbg->max_pages < pt_stride) return KV4_ERR_SHAPE;
    d = kv4::DecodeDebug{dbg->qcodes, dbg->qsum, dbg->qk, dbg->pcode, dbg->pv, dbg->max_ctx,
                         dbg->max_pages};
  }
  const kv4::DecodeWorkspace ws =
      kv4::carve_workspace(workspace, B, Hq, cache->num_kv_heads, nw);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (k_new && cache->window <= 0) {
    // no protected workgroup owns the new token: append first, then decode
    hipError_t e = kv4::launch_append(view(cache), static_cast<const uint16_t*>(k_new),
                                      static_cast<const uint16_t*>(v_new), pos_new, slot, page_table,
                                      pt_stride, B, st);
    if (e != hipSuccess) return hip_fail(e);
    k_new = v_new = nullptr;
    pos_new = nullptr;
  }
  hipError_t e = kv4::launch_decode(view(cache), static_cast<const uint16_t*>(q), ctx_len, slot,
                                    page_table, pt_stride, B, Hq, scale_log2(softmax_scale), out,
                                    lse, ws, dbg ? &d : nullptr, st, static_cast<hipEvent_t>(ev0),
                                    static_cast<hipEvent_t>(ev1), mx,
                                    static_cast<const uint16_t*>(k_new),
                                    static_cast<const uint16_t*>(v_new), pos_new);
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv4_decode_attention(const kv4_cache_desc* cache, const void* q, const int32_t* ctx_len,
                         const int32_t* slot, const int32_t* page_table, int32_t pt_stride,
                         int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale, float* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(cache, q, ctx_len, slot, page_table, pt_stride, B, Hq, max_ctx,
                       softmax_scale, out, lse, workspace, workspace_bytes, nullptr, stream);
}

int kv4_decode_attention_debug(const kv4_cache_desc* cache, const void* q,
                               const int32_t* ctx_len, const int32_t* slot,
                               const int32_t* page_table, int32_t pt_stride, int32_t B,
                               int32_t Hq, int32_t max_ctx, float softmax_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               const kv4_decode_debug* dbg, void* stream) {
  if (!dbg) return KV4_ERR_NULLPTR;
  return decode_common(cache, q, ctx_len, slot, page_table, pt_stride, B, Hq, max_ctx,
                       softmax_scale, out, lse, workspace, workspace_bytes, dbg, stream);
}

int kv4_append_decode_attention(const kv4_cache_desc* cache, const void* k, const void* v,
                                const int32_t* pos, const void* q, const int32_t* ctx_len,
                                const int32_t* slot, const int32_t* page_table, int32_t pt_stride,
                                int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!k || !v || !pos) return KV4_ERR_NULLPTR;
  return decode_common(cache, q, ctx_len, slot, page_table, pt_stride, B, Hq, max_ctx,
                       softmax_scale, out, lse, workspace, workspace_bytes, nullptr, stream, nullptr,
                       nullptr, false, k, v, pos);
}

int kv4_append_decode_attention_noalloc(const kv4_cache_desc* cache, const void* k, const void* v,
                                        const int32_t* pos, const void* q, const int32_t* ctx_len,
                                        const int32_t* slot, const int32_t* page_table,
                                        int32_t pt_stride, int32_t B, int32_t Hq, int32_t max_ctx,
                                        float softmax_scale, float* out, float* lse, void* stream) {
  if (!k || !v || !pos) return KV4_ERR_NULLPTR;
  // host-checkable errors first, so that a refused call touches no device state
  int rc = check_decode(cache, q, ctx_len, page_table, pt_stride, B, Hq, max_ctx, out, lse);
  if (rc != KV4_OK) return rc;
  if (B > 65535) return KV4_ERR_SHAPE;
  const size_t need = kv4::decode_workspace_bytes(B, Hq, cache->num_kv_heads, kv4::main_region_waves());
  if (need > KV4_NOALLOC_SCRATCH_BYTES) return KV4_ERR_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return KV4_ERR_HIP;
  // Nothing in the workspace has to start at zero: every partial, chunk range
  // and plan entry the merge reads is written earlier in the same step.
  return decode_common(cache, q, ctx_len, slot, page_table, pt_stride, B, Hq, max_ctx,
                       softmax_scale, out, lse, ws, KV4_NOALLOC_SCRATCH_BYTES, nullptr, stream,
                       nullptr, nullptr, false, k, v, pos);
}

int kv4bench_decode_attention_timed(const kv4_cache_desc* cache, const void* k, const void* v,
                                    const int32_t* pos, const void* q, const int32_t* ctx_len,
                                    const int32_t* slot, const int32_t* page_table,
                                    int32_t pt_stride, int32_t B, int32_t Hq, int32_t max_ctx,
                                    float softmax_scale, float* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* ev_main_begin, void* ev_main_end,
                                    void* stream) {
  if ((k == nullptr) != (v == nullptr) || (k == nullptr) != (pos == nullptr)) return KV4_ERR_NULLPTR;
  return decode_common(cache, q, ctx_len, slot, page_table, pt_stride, B, Hq, max_ctx,
                       softmax_scale, out, lse, workspace, workspace_bytes, nullptr, stream,
                       ev_main_begin, ev_main_end, false, k, v, pos);
}

size_t kv4bench_bf16_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_ctx) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_ctx <= 0) return 0;
  return kv4::bf16_workspace_bytes(B, Hq, Hkv, kv4::main_region_waves());
}

int kv4bench_bf16_paged_decode(const void* pages, int32_t num_pages, int32_t Hkv, const void* q,
                               const int32_t* ctx_len, const int32_t* page_table,
                               int32_t pt_stride, int32_t B, int32_t Hq, int32_t max_ctx,
                               float softmax_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!pages || !q || !ctx_len || !page_table || !out || !lse) return KV4_ERR_NULLPTR;
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || Hq / Hkv != kv4::GQA)
    return KV4_ERR_UNSUPPORTED;
  if (num_pages <= 0 || B <= 0 || B > 65535 || pt_stride <= 0 || max_ctx <= 0 ||
      static_cast<int64_t>(max_ctx) > static_cast<int64_t>(pt_stride) * 16)
    return KV4_ERR_SHAPE;
  const int nw = kv4::main_region_waves();
  if (!workspace || workspace_bytes < kv4::bf16_workspace_bytes(B, Hq, Hkv, nw))
    return KV4_ERR_WORKSPACE;
  hipError_t e = kv4::launch_bf16_decode(static_cast<const uint16_t*>(pages), num_pages, Hkv,
                                         static_cast<const uint16_t*>(q), ctx_len, page_table,
                                         pt_stride, B, Hq, scale_log2(softmax_scale), out, lse,
                                         workspace, nw, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

// ---- re-prefill attention ------------------------------------------------------

size_t kv4_prefill_attention_workspace_bytes(const kv4_cache_desc* cache, int32_t total_q,
                                             int32_t Hq, int32_t max_ctx) {
  if (check_cache(cache) != KV4_OK || total_q <= 0 || Hq <= 0 || Hq % cache->num_kv_heads != 0 ||
      max_ctx <= 0)
    return 0;
  return kv4::chunk_workspace_bytes(total_q, Hq, cache->num_kv_heads, kv4::main_region_waves());
}

static int chunk_common(const kv4_cache_desc* cache, const void* q, const int32_t* cu_seqlens,
                        const int32_t* start_pos, const int32_t* slot, const int32_t* page_table,
                        int32_t pt_stride, int32_t nseq, int32_t total_q, int32_t Hq, int32_t max_ctx,
                        float softmax_scale, float* out, float* lse, void* workspace,
                        size_t workspace_bytes, const kv4_decode_debug* dbg, void* stream) {
  int rc = check_cache(cache);
  if (rc != KV4_OK) return rc;
  if (!q || !cu_seqlens || !start_pos || !page_table || !out || !lse) return KV4_ERR_NULLPTR;
  const int Hkv = cache->num_kv_heads;
  if (Hq <= 0 || Hq % Hkv != 0) return KV4_ERR_UNSUPPORTED;
  if (nseq <= 0 || total_q <= 0 || pt_stride <= 0 || max_ctx <= 0 ||
      static_cast<int64_t>(max_ctx) > static_cast<int64_t>(pt_stride) * 16)
    return KV4_ERR_SHAPE;
  if (static_cast<int64_t>(total_q) * kv4::query_head_groups(Hq, Hkv) * (max_ctx / 16 + 1) > INT32_MAX)
    return KV4_ERR_SHAPE;
  const int nw = kv4::main_region_waves();
  if (!workspace || workspace_bytes < kv4::chunk_workspace_bytes(total_q, Hq, Hkv, nw))
    return KV4_ERR_WORKSPACE;
  kv4::DecodeDebug d{};
  if (dbg) {
    if (dbg->max_ctx < max_ctx || dbg->max_pages < pt_stride) return KV4_ERR_SHAPE;
    d = kv4::DecodeDebug{dbg->qcodes, dbg->qsum, dbg->qk, dbg->pcode, dbg->pv, dbg->max_ctx,
                         dbg->max_pages};
  }
  hipError_t e = kv4::launch_chunk_attention(view(cache), static_cast<const uint16_t*>(q), cu_seqlens,
                                             start_pos, nseq, total_q, slot, page_table, pt_stride, Hq,
                                             scale_log2(softmax_scale), out, lse, workspace, nw,
                                             dbg ? &d : nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv4_prefill_attention(const kv4_cache_desc* cache, const void* q, const int32_t* cu_seqlens,
                          const int32_t* start_pos, const int32_t* slot, const int32_t* page_table,
                          int32_t pt_stride, int32_t nseq, int32_t total_q, int32_t Hq,
                          int32_t max_ctx, float softmax_scale, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_common(cache, q, cu_seqlens, start_pos, slot, page_table, pt_stride, nseq, total_q,
                      Hq, max_ctx, softmax_scale, out, lse, workspace, workspace_bytes, nullptr, stream);
}

int kv4_prefill_attention_debug(const kv4_cache_desc* cache, const void* q,
                                const int32_t* cu_seqlens, const int32_t* start_pos,
                                const int32_t* slot, const int32_t* page_table, int32_t pt_stride,
                                int32_t nseq, int32_t total_q, int32_t Hq, int32_t max_ctx,
                                float softmax_scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, const kv4_decode_debug* dbg, void* stream) {
  if (!dbg) return KV4_ERR_NULLPTR;
  return chunk_common(cache, q, cu_seqlens, start_pos, slot, page_table, pt_stride, nseq, total_q,
                      Hq, max_ctx, softmax_scale, out, lse, workspace, workspace_bytes, dbg, stream);
}

// ---- MXFP4 variant -----------------------------------------------------------

int kv4mx_append(const kv4_cache_desc* cache, const void* k, const void* v, const int32_t* pos,
                 const int32_t* slot, const int32_t* page_table, int32_t pt_stride, int32_t B,
                 void* stream) {
  int rc = check_cache(cache);
  if (rc != KV4_OK) return rc;
  if (!k || !v || !pos || !page_table) return KV4_ERR_NULLPTR;
  if (B <= 0 || pt_stride <= 0 || B > 65535) return KV4_ERR_SHAPE;
  hipError_t e = kv4::launch_append(view(cache), static_cast<const uint16_t*>(k),
                                    static_cast<const uint16_t*>(v), pos, slot, page_table,
                                    pt_stride, B, static_cast<hipStream_t>(stream), true);
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv4mx_prefill_quantize(const kv4_cache_desc* cache, const void* k, const void* v,
                           const int32_t* cu_seqlens, const int32_t* start_pos, const int32_t* slot,
                           const int32_t* page_table, int32_t pt_stride, int32_t nseq,
                           int32_t max_seqlen, void* stream) {
  int rc = check_cache(cache);
  if (rc != KV4_OK) return rc;
  if (!k || !v || !cu_seqlens || !start_pos || !page_table) return KV4_ERR_NULLPTR;
  if (nseq <= 0 || nseq > 65535 || pt_stride <= 0 || max_seqlen <= 0) return KV4_ERR_SHAPE;
  hipError_t e = kv4::launch_prefill(view(cache), static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), cu_seqlens, start_pos, slot,
                                     page_table, pt_stride, nseq, max_seqlen,
                                     static_cast<hipStream_t>(stream), true);
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv4mx_decode_attention(const kv4_cache_desc* cache, const void* q, const int32_t* ctx_len,
                           const int32_t* slot, const int32_t* page_table, int32_t pt_stride,
                           int32_t B, int32_t Hq, int32_t max_ctx, float softmax_scale, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(cache, q, ctx_len, slot, page_table, pt_stride, B, Hq, max_ctx,
                       softmax_scale, out, lse, workspace, workspace_bytes, nullptr, stream, nullptr,
                       nullptr, true);
}

// ---- KV8 everywhere --------------------------------------------------------

static int check_kv8(const kv8_cache_desc* c) {
  if (!c) return KV4_ERR_NULLPTR;
  if (c->abi_version != KV4_ABI_VERSION || c->page_size != 16 || c->head_dim != 128)
    return KV4_ERR_UNSUPPORTED;
  if (c->num_pages <= 0 || c->num_kv_heads <= 0) return KV4_ERR_SHAPE;
  if (!c->pages) return KV4_ERR_NULLPTR;
  return KV4_OK;
}

int kv8_append(const kv8_cache_desc* cache, const void* k, const void* v, const int32_t* pos,
               const int32_t* page_table, int32_t pt_stride, int32_t B, void* stream) {
  int rc = check_kv8(cache);
  if (rc != KV4_OK) return rc;
  if (!k || !v || !pos || !page_table) return KV4_ERR_NULLPTR;
  if (B <= 0 || pt_stride <= 0 || B > 65535) return KV4_ERR_SHAPE;
  hipError_t e = kv4::launch_kv8_append(static_cast<uint8_t*>(cache->pages), cache->num_kv_heads,
                                        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                        pos, page_table, pt_stride, B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv8_prefill_quantize(const kv8_cache_desc* cache, const void* k, const void* v,
                         const int32_t* cu_seqlens, const int32_t* start_pos,
                         const int32_t* page_table, int32_t pt_stride, int32_t nseq,
                         int32_t max_seqlen, void* stream) {
  int rc = check_kv8(cache);
  if (rc != KV4_OK) return rc;
  if (!k || !v || !cu_seqlens || !start_pos || !page_table) return KV4_ERR_NULLPTR;
  if (nseq <= 0 || nseq > 65535 || pt_stride <= 0 || max_seqlen <= 0) return KV4_ERR_SHAPE;
  hipError_t e = kv4::launch_kv8_prefill(static_cast<uint8_t*>(cache->pages), cache->num_kv_heads,
                                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                         cu_seqlens, start_pos, page_table, pt_stride, nseq,
                                         max_seqlen, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

size_t kv8_decode_workspace_bytes(const kv8_cache_desc* cache, int32_t B, int32_t Hq,
                                  int32_t max_ctx) {
  if (check_kv8(cache) != KV4_OK || B <= 0 || Hq <= 0 || Hq % cache->num_kv_heads != 0 || max_ctx <= 0)
    return 0;
  return kv4::decode_workspace_bytes(B, Hq, cache->num_kv_heads, kv4::kv8_region_waves());
}

static int kv8_decode_common(const kv8_cache_desc* cache, const void* q, const int32_t* ctx_len,
                             const int32_t* page_table, int32_t pt_stride, int32_t B, int32_t Hq,
                             int32_t max_ctx, float softmax_scale, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, const kv4_decode_debug* dbg,
                             void* stream) {
  int rc = check_kv8(cache);
  if (rc != KV4_OK) return rc;
  if (!q || !ctx_len || !page_table || !out || !lse) return KV4_ERR_NULLPTR;
  const int Hkv = cache->num_kv_heads;
  if (Hq <= 0 || Hq % Hkv != 0) return KV4_ERR_UNSUPPORTED;
  if (B <= 0 || B > 65535 || pt_stride <= 0 || max_ctx <= 0 ||
      static_cast<int64_t>(max_ctx) > static_cast<int64_t>(pt_stride) * 16)
    return KV4_ERR_SHAPE;
  if (static_cast<int64_t>(B) * kv4::query_head_groups(Hq, Hkv) * (max_ctx / 16 + 1) > INT32_MAX)
    return KV4_ERR_SHAPE;
  const int nw = kv4::kv8_region_waves();
  if (!workspace || workspace_bytes < kv4::decode_workspace_bytes(B, Hq, Hkv, nw))
    return KV4_ERR_WORKSPACE;
  kv4::DecodeDebug d{};
  if (dbg) {
    if (dbg->max_ctx < max_ctx || dbg->max_pages < pt_stride) return KV4_ERR_SHAPE;
    d = kv4::DecodeDebug{dbg->qcodes, dbg->qsum, dbg->qk, nullptr, nullptr, dbg->max_ctx,
                         dbg->max_pages};
  }
  const kv4::DecodeWorkspace ws = kv4::carve_workspace(workspace, B, Hq, Hkv, nw);
  hipError_t e = kv4::launch_kv8_decode(static_cast<const uint8_t*>(cache->pages), Hkv,
                                        static_cast<const uint16_t*>(q), ctx_len, page_table,
                                        pt_stride, B, Hq, scale_log2(softmax_scale), out, lse, ws,
                                        dbg ? &d : nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV4_OK : hip_fail(e);
}

int kv8_decode_attention(const kv8_cache_desc* cache, const void* q, const int32_t* ctx_len,
                         const int32_t* page_table, int32_t pt_stride, int32_t B, int32_t Hq,
                         int32_t max_ctx, float softmax_scale, float* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return kv8_decode_common(cache, q, ctx_len, page_table, pt_stride, B, Hq, max_ctx, softmax_scale,
                           out, lse, workspace, workspace_bytes, nullptr, stream);
}

int kv8_decode_attention_debug(const kv8_cache_desc* cache, const void* q, const int32_t* ctx_len,
                               const int32_t* page_table, int32_t pt_stride, int32_t B,
                               int32_t Hq, int32_t max_ctx, float softmax_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               const kv4_decode_debug* dbg, void* stream) {
  if (!dbg) return KV4_ERR_NULLPTR;
  return kv8_decode_common(cache, q, ctx_len, page_table, pt_stride, B, Hq, max_ctx, softmax_scale,
                           out, lse, workspace, workspace_bytes, dbg, stream);
}

}  // extern "C"
