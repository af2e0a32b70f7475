// kv4_internal.hpp -- kernel launchers shared between the translation units of
// libkv4 (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kv4 {

struct CacheView {
  uint8_t* pages;
  int8_t* side_codes;
  uint16_t* side_scales;
  int num_pages, Hkv, max_slots;
  int sink, window;  // protection budget s, w (s % 16 == 0, s + w <= 144)
};

struct DecodeDebug {
  int8_t* qcodes;
  int32_t* qsum;
  int32_t* qk;
  uint8_t* pcode;
  int32_t* pv;
  int max_ctx, max_pages;
};

// Workspace carve-up of one decode call.
struct DecodeWorkspace {
  int32_t* plan;   // [B+1] prefix sums of (main pages x Hv) over sequences (B > 256 only)
  float* prot;     // [B][Hq][kPart] partials of the protected region
  int2* mrange;    // [B*Hv] first and last chunk holding pages of each segment (0, -1: none)
  float* parts;    // [slots][4][kPart] partials of the main region
  int n_waves;     // waves of the main-region grid
};
constexpr int kPart = 132;  // A[128], Z, l, 2 pad

// Query-head groups per sequence: each kv-head's G = Hq / Hkv query heads in
// groups of up to 4 (the row count of the kernels' operands).
inline int query_head_groups(int Hq, int Hkv) { return Hkv * ((Hq / Hkv + 3) / 4); }

// Waves per SIMD of the main-region grid; every wave of the grid is resident
// at once (the equal-chunk split assumes it).
#ifndef KV4_MAIN_WAVES_PER_SIMD
#define KV4_MAIN_WAVES_PER_SIMD 4
#endif
// The KV8-everywhere instantiation holds more operands per wave (138 VGPRs)
// and runs 3 waves per SIMD.
#ifndef KV8_MAIN_WAVES_PER_SIMD
#define KV8_MAIN_WAVES_PER_SIMD 3
#endif

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int n_waves);
DecodeWorkspace carve_workspace(void* base, int B, int Hq, int Hkv, int n_waves);
int main_region_waves();  // size of the main-region grid on the current device
int kv8_region_waves();   // the same for the KV8-everywhere instantiation

// mx: write the main-region entry in the MXFP4 variant's format instead of INT4
hipError_t launch_append(const CacheView& c, const uint16_t* k, const uint16_t* v,
                         const int32_t* pos, const int32_t* slot, const int32_t* page_table,
                         int pt_stride, int B, hipStream_t s, bool mx = false);
hipError_t launch_prefill(const CacheView& c, const uint16_t* k, const uint16_t* v,
                          const int32_t* cu, const int32_t* start, const int32_t* slot,
                          const int32_t* page_table, int pt_stride, int nseq, int max_seqlen,
                          hipStream_t s, bool mx = false);
hipError_t launch_kv8_append(uint8_t* pages, int Hkv, const uint16_t* k, const uint16_t* v,
                             const int32_t* pos, const int32_t* page_table, int pt_stride, int B,
                             hipStream_t s);
hipError_t launch_kv8_prefill(uint8_t* pages, int Hkv, const uint16_t* k, const uint16_t* v,
                              const int32_t* cu, const int32_t* start, const int32_t* page_table,
                              int pt_stride, int nseq, int max_seqlen, hipStream_t s);
// KV8-everywhere decode: the main kernel's plan and pipeline over every page,
// no protected region (workspace as for launch_decode)
hipError_t launch_kv8_decode(const uint8_t* pages, int Hkv, const uint16_t* q, const int32_t* ctx,
                             const int32_t* page_table, int pt_stride, int B, int Hq,
                             float scale_log2, float* out, float* lse, const DecodeWorkspace& ws,
                             const DecodeDebug* dbg, hipStream_t s);
hipError_t launch_decode(const CacheView& c, const uint16_t* q, const int32_t* ctx,
                         const int32_t* slot, const int32_t* page_table, int pt_stride, int B,
                         int Hq, float scale_log2, float* out, float* lse,
                         const DecodeWorkspace& ws, const DecodeDebug* dbg, hipStream_t s,
                         hipEvent_t ev_main_begin = nullptr, hipEvent_t ev_main_end = nullptr,
                         bool mx = false, const uint16_t* k_new = nullptr,
                         const uint16_t* v_new = nullptr, const int32_t* pos_new = nullptr);
// Re-prefill (chunked-prefill) attention: query-blocked (blocks of 8 tokens
// per kv-head workgroup) over the protected rows and the main region, merged
// in the kernel; the workspace holds the block bases.
size_t chunk_workspace_bytes(int T, int Hq, int Hkv, int n_waves);
hipError_t launch_chunk_attention(const CacheView& c, const uint16_t* q, const int32_t* cu,
                                  const int32_t* start, int nseq, int T, const int32_t* slot,
                                  const int32_t* page_table, int pt_stride, int Hq, float scale_log2,
                                  float* out, float* lse, void* ws_base, int n_waves,
                                  const DecodeDebug* dbg, hipStream_t s);
hipError_t launch_prefill_blocked(const CacheView& c, const uint16_t* q, const int32_t* cu,
                                  const int32_t* start, int nseq, int T, const int32_t* slot,
                                  const int32_t* page_table, int pt_stride, int Hq, float scale_log2,
                                  float* out, float* lse, int32_t* blk_base, const DecodeDebug* dbg,
                                  hipStream_t s);
hipError_t launch_bf16_decode(const uint16_t* pages, int num_pages, int Hkv, const uint16_t* q,
                              const int32_t* ctx, const int32_t* page_table, int pt_stride, int B,
                              int Hq, float scale_log2, float* out, float* lse, void* ws,
                              int n_waves, hipStream_t s);
size_t bf16_workspace_bytes(int B, int Hq, int Hkv, int n_waves);

}  // namespace kv4
