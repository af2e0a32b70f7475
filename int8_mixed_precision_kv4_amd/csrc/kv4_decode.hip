// kv4_decode.hip -- one decode step of KV4-RL hybrid attention
// (paper.rainbus.top summary, "方法步骤详情" step 4 and "核心方法"; onedev.kr
// summary, "전제와 한계").
//
// Two launches on the caller's stream (three for more than 256 sequences,
// when a one-workgroup plan_kernel first writes the work plan):
//   1. main_kernel.  Its first workgroups are a fixed set of independent
//      waves: the concatenated list of main-region pages of all (sequence,
//      query-head group) segments is cut into equal contiguous chunks, one
//      per wave (split-K with exact load balance); each wave builds the plan
//      (prefix sums of main pages) in registers and rotates / INT8-quantizes
//      the (up to) 4 queries of each group it visits.  Per page: integer QK on MFMA (INT8
//      query x unpacked INT4 keys), delta/m applied after the dot, tile
//      softmax, INT8 P operand with the V scale folded in, integer PV on
//      MFMA, FP32 running merge; a wave writes one partial per segment it
//      touches.  Its last B*Hv workgroups compute the protected region of one
//      (sequence, query-head group) each (INT8 QK against the side keys, FP32 softmax,
//      PV over BF16-dequantized side values); they are dispatched as the
//      main-region waves retire, so they run in the main region's tail.
//   2. merge_kernel, one workgroup per (query-head group, sequence): exact
//      log-sum-exp merge of the protected partial with the main partials,
//      written as out and lse.
#include <type_traits>

#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace kv4 {
namespace {

struct DecArgs {
  const uint8_t* pages;
  const int8_t* side_codes;
  const uint16_t* side_scales;
  int Hkv, Hq, B;
  // query-head groups: each kv-head's G = Hq / Hkv query heads form R =
  // ceil(G / 4) groups of up to 4 (the rows of the kernels' operands), Hv =
  // Hkv * R groups per sequence
  int G, R, Hv;
  const uint32_t* q;  // bf16 pairs
  const int32_t* ctx;
  const int32_t* slot;
  const int32_t* page_table;
  int pt_stride;
  // Fused append (decode step only): this step's token of sequence b at
  // position pos_new[b] (= ctx[b] - 1), bf16 pairs [B][Hkv][64]; NULL: none.
  // Its protected workgroup writes the token's page entry and side row before
  // attending (the token is in the recent window, so nothing else reads it).
  const uint32_t* k_new;
  const uint32_t* v_new;
  const int32_t* pos_new;
  int sink, window;  // protection budget s, w
  float scale_log2;
  float* out;
  float* lse;
  DecodeWorkspace ws;
  DecodeDebug dbg;
};

// Query-head group v (0 <= v < Hv) of a sequence: kv-head gp = v / R and
// query heads h0 .. h0 + nh - 1 (nh = 4 except in the last group of a kv-head
// when G is not a multiple of 4).  The kernels compute all 4 rows of a group;
// the rows past nh repeat head h0 + nh - 1 and are never stored.
struct HeadGroup {
  int gp, h0, nh;
};
__device__ __forceinline__ HeadGroup head_group(const DecArgs& a, int v) {
  if (a.R == 1) return HeadGroup{v, v * a.G, a.G};  // G <= 4: one group per kv-head
  const int gp = v / a.R, k = v - gp * a.R;
  return HeadGroup{gp, gp * a.G + 4 * k, min(4, a.G - 4 * k)};
}

// Main region of a query attending [0, L) of a cache that ends at E (E = L
// for a decode step): M = [s, min(L, E-w)), logical pages s/16 .. (end-1)/16
// (s is a multiple of 16, so the first page starts at s).
__device__ __forceinline__ int main_end_of(int L, int E, int w) { return min(L, E - w); }
__device__ __forceinline__ int main_pages(int L, int E, int s, int w) {
  const int me = main_end_of(L, E, w);
  return me > s ? (me - 1) / PAGE - s / PAGE + 1 : 0;
}

// plan[b] = sum over earlier sequences of main_pages * Hv (one workgroup).
__device__ void build_plan(const DecArgs& a) {
  __shared__ int32_t scan[256];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) {
    carry = 0;
    a.ws.plan[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < a.B; base += 256) {
    const int b = base + threadIdx.x;
    scan[threadIdx.x] = (b < a.B) ? main_pages(a.ctx[b], a.ctx[b], a.sink,
                                               a.window) * a.Hv : 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int t = (threadIdx.x >= off) ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += t;
      __syncthreads();
    }
    if (b < a.B) a.ws.plan[b + 1] = carry + scan[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 255) carry += scan[255];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- query --

typedef int v4i __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) uint8_t* gptr;
typedef __attribute__((address_space(3))) void* lptr;

// s_waitcnt encodings (gfx9): all vector-memory loads (including direct-to-LDS
// loads) landed; all LDS reads returned.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// Cache policy of the page loads: non-temporal.  Every page block of a step is
// read once, so the loads stream past the caches instead of allocating in
// them (about 10% faster for the whole main kernel than default loads).
constexpr int kNT = 2;
// Word 3 of a buffer resource on gfx9 (32-bit data format, no swizzle): a raw
// buffer load past num_records returns zeros.
constexpr int kBufferWord3 = 0x00020000;

// Plan for batches of more than 256 sequences (smaller batches build it in
// registers in every main-kernel wave): one workgroup.
__global__ __launch_bounds__(256) void plan_kernel(DecArgs a) { build_plan(a); }

// Row-of-16 reductions of an int (lanes 16r .. 16r+15).
__device__ __forceinline__ int row16_sum_i(int v) {
  v += xor_lane_i<1>(v);
  v += xor_lane_i<2>(v);
  v += xor_lane_i<4>(v);
  return v + xor_lane_i<8>(v);
}

// Rotated INT8 query of the 4 heads of a group, computed by one wave: lane
// (head grp, r16) holds channels 8 r16 .. 8 r16 + 7 (raw = their BF16 values).
// FWHT strides 1, 2, 4 inside the lane, then 8, 16, 32, 64 across lanes (xor
// 1, 2, 4, 8 within the row of 16), in that order, then the 2^-3.5 scale;
// s_q = max|x| / 127, codes = clamp(rint(x / s_q)), S_q = their sum.
struct GroupQuery {
  int c[8];
  float c_q;
  int S;
};
__device__ __forceinline__ void rotate_group_query(uint4 raw, int r16, float x[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
  fwht128_row16(x, r16);
}
__device__ __forceinline__ GroupQuery quantize_group_query(uint4 raw, float scale_log2, int r16) {
  float x[8];
  rotate_group_query(raw, r16, x);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = row16_max(amax);
  const float s_q = amax / 127.0f;
  GroupQuery g;
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g.c[j] = s_q != 0.0f ? static_cast<int>(fminf(fmaxf(__builtin_rintf(x[j] / s_q), -127.0f), 127.0f)) : 0;
    sum += g.c[j];
  }
  g.S = row16_sum_i(sum);
  g.c_q = s_q * scale_log2;  // c_q: s_q, the scale and log2(e)
  return g;
}

// QK on a 16x16 MFMA with the 4 heads' query rows each repeated 4 times
// (A row r = head r / 4): lane l then receives rows 4 (l / 16) .. + 3 of
// column l % 16, all four the dot product of head l / 16 with position
// l % 16, which is the (head, position) layout of the softmax work; no lane
// moves are needed.
__device__ __forceinline__ int qk_rows(v4i d) { return d[0]; }

// ------------------------------------------------------------ protected --

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Two FP32 values as packed BF16 (nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{x, y}), b2));
}

// Protected-region partial of one (query-head group v, sequence b), computed by
// one workgroup of the main kernel (the last B*Hv workgroups of its grid, which
// the dispatcher starts as main-region workgroups retire; none when s = w = 0).
// Only rows [0, s+w) are read.  QK: up to 9 MFMA row groups of 16 side rows
// spread over the 4 waves.  Softmax: wave h for head h, its FP32 weights
// written to LDS as two BF16 parts, hi = bf16(e) and lo = bf16(e - hi), 16
// significant bits.  PV on BF16 MFMAs over the V rows staged in LDS (v^ =
// bf16(s_v c)): wave w owns channels 32 w .. 32 w + 31 for all rows and heads,
// so each wave stores its share of the partial directly; wave h adds Z and l
// of head h.
constexpr int kPvRows = 160;  // 144 side rows padded to 5 MFMA k-steps of 32
constexpr int kPrSe = 0;                                 // float [144][4] logits
constexpr int kPrSv = kPrSe + SIDE_ROWS * GQA * 4;       // float [160] V scales (0: row unused)
constexpr int kPrP = kPrSv + kPvRows * 4;                // bf16 [2][4][160] weights, hi then lo
constexpr int kPrV = kPrP + 2 * GQA * kPvRows * 2;       // int8 [144][128] V codes of the side rows
constexpr int kPrQ = kPrV + SIDE_ROWS * HD;              // int8 [4][128] query codes
constexpr int kPrC = kPrQ + GQA * HD;                    // float [4] c_q per head
constexpr int kProtLds = kPrC + GQA * 4;                 // 24192 B
constexpr int kProtLdsFused = kProtLds + 2 * HD + 8;     // plus this step's INT8 row and its scales
// The PV reads of rows 144 .. 159 land in the bytes after the V rows (finite
// int8 values, weighted by a zero scale): they must stay inside the role's LDS.
static_assert(kPrV + kPvRows * HD <= kProtLdsFused + 2048, "padded V rows inside the protected LDS");

template <bool DEBUG>
__device__ __forceinline__ void protected_partial(const DecArgs& a, int v, int b, uint8_t* lds_raw) {
  const int wave = wave_id(), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int r16 = lane & 15, grp = lane >> 4;
  auto se = reinterpret_cast<float (*)[GQA]>(lds_raw + kPrSe);
  float* ssv = reinterpret_cast<float*>(lds_raw + kPrSv);
  uint16_t* pw = reinterpret_cast<uint16_t*>(lds_raw + kPrP);  // [hi, lo][head][160]
  uint8_t* vst = lds_raw + kPrV;
  int8_t* qn = reinterpret_cast<int8_t*>(lds_raw + kPrQ);
  float* cqs = reinterpret_cast<float*>(lds_raw + kPrC);

  // ---- every load is issued before anything waits on one: the scalar
  // lookups, this step's token (fused append) and the query, then the side
  // rows (K into registers, V into LDS) and their scales as raw bits.  Values
  // are converted only after the last load has gone out, so that the phase is
  // one round trip (plus the slot and page-table lookups it depends on) instead
  // of a chain of them.  Wave 0 makes the INT8 row, wave 1 the INT4 K half of
  // the page entry, wave 2 its V half.  Only the kv-head's first query-head
  // group writes them; every group makes the INT8 row for itself (the side row
  // it loads may be read before that write).
  const int L = ld_const(a.ctx + b);
  const int E = L;  // the cache ends at this step's token
  const int sq = b;
  const int slot = a.slot ? ld_const(a.slot + sq) : sq;
  const int new_pos = a.k_new ? ld_const(a.pos_new + b) : 0;
  const HeadGroup hg = head_group(a, v);  // wave h: query head hg.h0 + h (h < hg.nh)
  const int g = hg.gp;
  const size_t qb = static_cast<size_t>(b) * a.Hq + hg.h0;
  const size_t bh = qb + min(wave, hg.nh - 1);  // the query of head `wave`
  const uint32_t qw = a.q[bh * 64 + lane];
  const bool writer = hg.h0 == g * a.G;
  uint32_t kw = 0, vw = 0;
  if (a.k_new) {
    const size_t vec = static_cast<size_t>(b) * a.Hkv + g;
    if (wave == 0 || (writer && wave == 1)) kw = a.k_new[vec * 64 + lane];
    if (wave == 0 || (writer && wave == 2)) vw = a.v_new[vec * 64 + lane];
  }
  // rows that can hold a position of the region: the sinks below L, and the
  // ring when the window [max(s, L - w), L) is not empty
  const int nrows = L > max(a.sink, E - a.window) ? a.sink + a.window : min(a.sink, L);
  const size_t row0 = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS;
  const gptr side = (gptr)a.side_codes + row0 * 2 * HD;
  // The K rows and scales as buffers of nrows rows: a load of a row past
  // nrows returns zeros and touches no memory, so these loads need no branch
  // (a branch around a load lets the compiler wait for it at the join, which
  // made the row groups dependent round trips).
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.side_codes) + row0 * 2 * HD, 0, nrows * 2 * HD,
                                        kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.side_scales) + row0 * 2, 0, nrows * 4,
                                        kBufferWord3);
  // K operands and scale bits of this wave's row groups (rg = wave + 4k; row
  // groups past the 9 of the buffer read as zeros)
  v4i kop[3][2];
  uint32_t skr[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int row = 16 * (wave + 4 * k) + r16;
    kop[k][0] = __builtin_amdgcn_raw_buffer_load_b128(krs, row * 2 * HD + 16 * grp, 0, kNT);
    kop[k][1] = __builtin_amdgcn_raw_buffer_load_b128(krs, row * 2 * HD + 64 + 16 * grp, 0, kNT);
    skr[k] = __builtin_amdgcn_raw_buffer_load_b16(srs, 4 * row, 0, kNT);
  }
  // V scale bits of row tid (selected away below for a row outside the region)
  const uint32_t svr = __builtin_amdgcn_raw_buffer_load_b16(srs, 4 * tid + 2, 0, kNT);
  // V codes of the used rows into LDS, 8 rows (1 KB) per instruction: lane l
  // moves bytes 16 (l % 8) .. of row 8 j + l / 8 (blocks j = wave, wave + 4, ..)
  for (int j = wave; 8 * j < nrows; j += 4) {
    const int r = 8 * j + (lane >> 3);
    __builtin_amdgcn_global_load_lds(side + (2 * r + 1) * HD + 16 * (lane & 7), (lptr)(vst + 1024 * j), 16, 0,
                                     kNT);
  }
  // the page slot of this step's token (writer waves 1 and 2), then the two
  // V bytes that wave 2 rewrites around its nibble
  int r_new = -1;
  uint8_t* new_blk = nullptr;
  uint32_t vb0 = 0, vb1 = 0;
  if (a.k_new) {
    r_new = new_pos < a.sink ? new_pos : a.sink + new_pos % a.window;  // w > 0 on this path
    if (writer && (wave == 1 || wave == 2)) {
      const int phys = ld_const(a.page_table + static_cast<size_t>(sq) * a.pt_stride + (new_pos >> 4));
      new_blk = const_cast<uint8_t*>(a.pages) + (static_cast<size_t>(phys) * a.Hkv + g) * BLOCK_BYTES;
      if (wave == 2) {
        const uint8_t* vb = new_blk + OFF_VCODE + 8 * (2 * lane) + ((new_pos & (PAGE - 1)) >> 1);
        vb0 = vb[0];
        vb1 = vb[8];
      }
    }
  }
  // ---- arithmetic on what arrives: the query first, then this step's token
  // Query of head `wave`: rotate like the keys, then symmetric INT8 with an
  // FP32 scale (lane l holds channels 2l, 2l+1); codes in natural order to LDS.
  {
    float x0 = bf16_lo(qw), x1 = bf16_hi(qw);
    fwht128_wave(x0, x1);
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const float s_q = amax / 127.0f;
    int c0 = 0, c1 = 0;
    if (s_q != 0.0f) {
      c0 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x0 / s_q), -127.0f), 127.0f));
      c1 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x1 / s_q), -127.0f), 127.0f));
    }
    reinterpret_cast<uint16_t*>(qn + wave * HD)[lane] = static_cast<uint16_t>((c0 & 0xFF) | ((c1 & 0xFF) << 8));
    if (lane == 0) cqs[wave] = s_q * a.scale_log2;
    if (DEBUG && wave < hg.nh) {
      const int S = wave_sum_i(c0 + c1);
      if (a.dbg.qsum && lane == 0) a.dbg.qsum[bh] = S;
      if (a.dbg.qcodes) {
        a.dbg.qcodes[bh * HD + 2 * lane] = static_cast<int8_t>(c0);
        a.dbg.qcodes[bh * HD + 2 * lane + 1] = static_cast<int8_t>(c1);
      }
    }
  }
  // Fused append: this step's token goes to its page slot and its side row,
  // and the INT8 row also to LDS; after the barrier below every wave replaces
  // what it loaded for that row (the loads above may have seen the old row).
  int8_t* nrow = reinterpret_cast<int8_t*>(lds_raw + kProtLds);   // [2][128] K, V codes
  float* nscale = reinterpret_cast<float*>(lds_raw + kProtLds + 2 * HD);  // s_k, s_v
  if (r_new >= 0 && (wave == 0 || (writer && wave < 3))) {
    const int t = new_pos & (PAGE - 1);
    float k0 = bf16_lo(kw), k1 = bf16_hi(kw);
    const float v0 = bf16_lo(vw), v1 = bf16_hi(vw);
    if (wave != 2) fwht128_wave(k0, k1);
    if (wave == 0) {
      const size_t rr = row0 + r_new;
      const Int8Row nr = make_int8_row(k0, k1, v0, v1);
      if (writer) store_int8_row(const_cast<int8_t*>(a.side_codes) + rr * 2 * HD,
                                 const_cast<uint16_t*>(a.side_scales) + rr * 2, nr, lane);
      reinterpret_cast<uint16_t*>(nrow)[lane] = static_cast<uint16_t>(nr.kp);
      reinterpret_cast<uint16_t*>(nrow)[64 + lane] = static_cast<uint16_t>(nr.vp);
      if (lane == 0) {
        nscale[0] = f16_value(nr.ks16);
        nscale[1] = f16_value(nr.vs16);
      }
    } else if (wave == 1) {
      write_int4_k(new_blk, t, k0, k1, lane);
    } else {
      write_int4_v(new_blk, t, v0, v1, lane, VBytes{static_cast<uint8_t>(vb0), static_cast<uint8_t>(vb1)});
    }
  }
  float sk[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sk[k] = f16_value(skr[k]);
  if (tid < kPvRows)
    ssv[tid] = tid < SIDE_ROWS && side_position(tid, L, E, a.sink, a.window) >= 0 ? f16_value(svr) : 0.0f;
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the staged V rows have landed
  __syncthreads();
  if (r_new >= 0) {  // this step's row from LDS, one read per lane, selected in place
    const v4i kn0 = *reinterpret_cast<const v4i*>(nrow + 16 * grp);
    const v4i kn1 = *reinterpret_cast<const v4i*>(nrow + 64 + 16 * grp);
    const float skn = nscale[0];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const bool hit = 16 * (wave + 4 * k) + r16 == r_new;
      kop[k][0] = hit ? kn0 : kop[k][0];
      kop[k][1] = hit ? kn1 : kop[k][1];
      sk[k] = hit ? skn : sk[k];
    }
    // the staged V row: read by the PV phase, after two more barriers
    if (wave == 0) reinterpret_cast<uint16_t*>(vst + r_new * HD)[lane] = reinterpret_cast<const uint16_t*>(nrow + HD)[lane];
    if (tid == r_new) ssv[tid] = nscale[1];
  }
  // A operand: row r16 = head r16 / 4 (each head's codes in four rows)
  v4i qa[2];
  qa[0] = *reinterpret_cast<const v4i*>(qn + (r16 >> 2) * HD + 16 * grp);
  qa[1] = *reinterpret_cast<const v4i*>(qn + (r16 >> 2) * HD + 64 + 16 * grp);
  const float c_q = cqs[grp];

  // ---- INT8 QK: lane (head grp, row 16 rg + r16)
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int rg = wave + 4 * k;
    if (rg < SIDE_ROWS / 16) {
      v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], kop[k][0], v4i{0, 0, 0, 0}, 0, 0, 0);
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], kop[k][1], d, 0, 0, 0);
      const int D8 = qk_rows(d);
      const int r = 16 * rg + r16;
      const int p = side_position(r, L, E, a.sink, a.window);
      se[r][grp] = (p >= 0) ? (static_cast<float>(D8) * sk[k]) * c_q : -INFINITY;
      if (DEBUG && a.dbg.qk && p >= 0 && grp < hg.nh) a.dbg.qk[(qb + grp) * a.dbg.max_ctx + p] = D8;
    }
  }
  __syncthreads();

  // ---- FP32 softmax of head `wave` over the region (rows not in use: 0); the
  // weights go to LDS as hi + lo BF16 parts, zero past row 144
  float zl = -INFINITY;
  for (int i = lane; i < SIDE_ROWS; i += 64) zl = fmaxf(zl, se[i][wave]);
  const float Z = wave_max(zl);
  float ls = 0.0f;
  for (int i = lane; i < kPvRows; i += 64) {
    const float e = i < SIDE_ROWS ? exp2s(se[i][wave] - Z) : 0.0f;
    ls += e;
    const uint32_t hi = pack_bf16x2(e, 0.0f) & 0xFFFFu;
    const uint32_t lo = pack_bf16x2(e - __uint_as_float(hi << 16), 0.0f) & 0xFFFFu;
    pw[wave * kPvRows + i] = static_cast<uint16_t>(hi);
    pw[(GQA + wave) * kPvRows + i] = static_cast<uint16_t>(lo);
  }
  ls = wave_sum(ls);
  __syncthreads();

  // ---- PV with v^ = bf16(s_v c): wave w, channels 32 w + 16 cb + n (column
  // blocks cb = 0, 1).  MFMA rows 4 cb + h carry head h's weights (A zero in
  // the other rows), so one accumulator gathers both blocks: lane (n, rg)
  // ends with rows 4 rg .. 4 rg + 3 = heads 0..3 of channel 32 w + 16 rg + n.
  // k = 32 rows per step, lane group grp holding rows 8 grp .. 8 grp + 7.
  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 zero4 = u4{0u, 0u, 0u, 0u};
  const int hrow = r16 & 3, blk = r16 >> 2;
#pragma unroll
  for (int st = 0; st < kPvRows / 32; ++st) {
    const int p0 = 32 * st + 8 * grp;
    const u4 ph = *reinterpret_cast<const u4*>(pw + hrow * kPvRows + p0);
    const u4 pl = *reinterpret_cast<const u4*>(pw + (GQA + hrow) * kPvRows + p0);
    const float4 sv0 = *reinterpret_cast<const float4*>(ssv + p0);
    const float4 sv1 = *reinterpret_cast<const float4*>(ssv + p0 + 4);
    const float sv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int ch = 32 * wave + 16 * cb + r16;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = sv[i] * static_cast<float>(reinterpret_cast<const int8_t*>(vst)[(p0 + i) * HD + ch]);
      const u4 pk = u4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7])};
      const v8bf vb = __builtin_bit_cast(v8bf, pk);
      const bool mine = blk == cb;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, mine ? ph : zero4), vb, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, mine ? pl : zero4), vb, acc, 0, 0, 0);
    }
  }
  // ---- this wave's 32 channels of the 4 heads' partials; Z and l of head `wave`
  if (grp < 2) {
#pragma unroll
    for (int h = 0; h < GQA; ++h)
      if (h < hg.nh) a.ws.prot[(qb + h) * kPart + 32 * wave + 16 * grp + r16] = acc[h];
  }
  if (lane == 0 && wave < hg.nh) {
    float* P = a.ws.prot + (qb + wave) * kPart;
    P[128] = Z;
    P[129] = ls;
  }
}

// ------------------------------------------------------------------ main --

__device__ __forceinline__ uint32_t lo_nibbles(uint32_t x) { return x & 0x0F0F0F0Fu; }
__device__ __forceinline__ v4i nib_lo(uint4 x) {
  return v4i{static_cast<int>(lo_nibbles(x.x)), static_cast<int>(lo_nibbles(x.y)),
             static_cast<int>(lo_nibbles(x.z)), static_cast<int>(lo_nibbles(x.w))};
}
// high nibbles of two dwords with one 64-bit shift
__device__ __forceinline__ uint64_t hi_nibbles64(uint32_t a, uint32_t b) {
  return ((static_cast<uint64_t>(b) << 32 | a) >> 4) & 0x0F0F0F0F0F0F0F0Full;
}
__device__ __forceinline__ v4i nib_hi(uint4 x) {
  const uint64_t h0 = hi_nibbles64(x.x, x.y), h1 = hi_nibbles64(x.z, x.w);
  return v4i{static_cast<int>(h0), static_cast<int>(h0 >> 32), static_cast<int>(h1), static_cast<int>(h1 >> 32)};
}
// 16 positions of one channel (8 nibble bytes) -> 16 INT8 operand bytes; byte
// i of the result holds position 8(i/8) + 2(i%4) + (i/4)%2.
__device__ __forceinline__ v4i nib_positions(uint32_t lo8, uint32_t hi8) {
  const uint64_t h = hi_nibbles64(lo8, hi8);
  return v4i{static_cast<int>(lo_nibbles(lo8)), static_cast<int>(h), static_cast<int>(lo_nibbles(hi8)),
             static_cast<int>(h >> 32)};
}
// inverse of that byte order
__device__ __forceinline__ int pcode_slot(int t) { return 8 * (t >> 3) + 4 * (t & 1) + ((t & 7) >> 1); }


// Per-wave LDS staging slot of one quad (4 pages of one segment):
//   [0, 4096)     K codes, tile t at 1024 t + 16 lane
//   [4096, 8192)  V codes, tile t at 4096 + 1024 t + 16 lane (lane (r16, g):
//                 the channel pair 4 r16 + g, i.e. channels 8 r16 + 2 g, + 1)
//   [8192, 8704)  metadata, page t at 8192 + 128 t: 16 x {delta, m} K, then V
// followed by 256 B where the P operand is assembled and 512 B where the
// query codes of a group are rearranged into the MFMA operand order.
constexpr int kSlotK = 0, kSlotV = 4096, kSlotMeta = 8192, kSlotP = 8704, kSlotQ = 8960, kQuadSlotBytes = 9472;

struct QuadRegs {
  uint4 kq[4], vq[4];
  uint32_t km[4], vm[4];
};

// Issue the direct-to-LDS loads of one quad.  Tile t reads physical page
// blk[t]; lane (r16, grp) fetches bytes 64 r16 + 16 grp of the tile's K codes
// and of its V codes (1 KB contiguous per instruction for both).  Tiles
// t >= np (past the piece's last page) are not loaded: the slot keeps whatever
// it held, and the compute masks those tiles by position (logit -inf, V
// metadata zero, P codes 0), which no bit pattern of theirs can undo, since
// their codes only meet P codes of 0 in the integer products.
__device__ __forceinline__ void quad_to_lds(uint8_t* slot, const gptr blk[4], int np, int lane, int r16,
                                            int grp) {
  const int koff = 64 * r16 + 16 * grp;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (t < np)
      __builtin_amdgcn_global_load_lds(blk[t] + koff, (lptr)(slot + kSlotK + 1024 * t), 16, 0, kNT);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (t < np)
      __builtin_amdgcn_global_load_lds(blk[t] + OFF_VCODE + koff, (lptr)(slot + kSlotV + 1024 * t), 16, 0, kNT);
  if (lane < 8 * np) {  // np pages x 128 B of metadata
    const int t = lane >> 3;
    const gptr mb = t == 0 ? blk[0] : t == 1 ? blk[1] : t == 2 ? blk[2] : blk[3];
    __builtin_amdgcn_global_load_lds(mb + OFF_KMETA + 16 * (lane & 7), (lptr)(slot + kSlotMeta), 16, 0, kNT);
  }
}

__device__ __forceinline__ void quad_from_lds(QuadRegs& q, const uint8_t* slot, int lane, int r16) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    q.kq[t] = *reinterpret_cast<const uint4*>(slot + kSlotK + 1024 * t + 16 * lane);
    // channel pair 4 r16 + t of tile grp (the k-group of the PV MFMA): channels 8 r16 + 2 t, + 1
    q.vq[t] = *reinterpret_cast<const uint4*>(slot + kSlotV + 1024 * (lane >> 4) + 256 * t + 16 * r16);
    q.km[t] = *reinterpret_cast<const uint32_t*>(slot + kSlotMeta + 128 * t + 4 * r16);
    q.vm[t] = *reinterpret_cast<const uint32_t*>(slot + kSlotMeta + 128 * t + 64 + 4 * r16);
  }
}


struct MainState {
  float Zr, Ls, Ms;
  float O[8];
};

// One quad of 4 tiles (pages) for the 4 heads of a group.  Lane = (head grp,
// position r16) for the softmax; MFMA operand layouts as described above.
// A position outside the region gets the logit -inf (so its weight is 0)
// and a zero V metadata word (so its u and e m_v are +0): two selects per
// tile, no branches.
template <bool DEBUG>
__device__ __forceinline__ void compute_quad(const DecArgs& a, MainState& st, const QuadRegs& q,
                                             int np, v4i qa0, v4i qa1, float c_q, float S_q,
                                             int j0, int main_end, size_t qb, int nh, uint8_t* stage,
                                             int r16, int grp, int pslot) {
  // integer QK of the four tiles
  v4i d[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa0, nib_lo(q.kq[t]), v4i{0, 0, 0, 0}, 0, 0, 0);
    d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa1, nib_hi(q.kq[t]), d[t], 0, 0, 0);
  }
  float zmax[4], e[4], u[4], umax[4], emv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int D = qk_rows(d[t]);
    const int pos = PAGE * (j0 + t) + r16;
    const bool valid = pos < (t < np ? main_end : 0);
    const float dk = f16_value(q.km[t] & 0xFFFFu);
    // q.k^ = s_q (delta * sum(qc*c) + m * sum(qc)); c_q carries s_q, the scale and log2(e)
    const float z0 = __builtin_fmaf(dk, static_cast<float>(D), mul_f16(S_q, q.km[t] >> 16)) * c_q;
    const float z = valid ? z0 : -INFINITY;
    zmax[t] = row16_max_ord(z);
    // a masked position: exp2s(-inf - zmax) = 0 (NaN when the whole tile is
    // masked, which exp2s also maps to 0); its metadata, which may be any
    // bits, is replaced by zeros
    e[t] = exp2s(z - zmax[t]);
    const uint32_t vmt = valid ? q.vm[t] : 0u;
    u[t] = mul_f16(e[t], vmt & 0xFFFFu);  // V scale folded into P
    emv[t] = mul_f16(e[t], vmt >> 16);    // V offset applied after the dot
    umax[t] = __uint_as_float(row16_max_u32(__float_as_uint(u[t])));
    if (DEBUG && valid && a.dbg.qk && grp < nh) a.dbg.qk[(qb + grp) * a.dbg.max_ctx + pos] = D;
    __builtin_amdgcn_sched_barrier(0);  // one tile at a time: keeps the register count under 128
  }
  // 127 / u_max of the 16 (tile, head) pairs with one IEEE division:
  // lane (h, r16) divides for tile r16 % 4, then quads broadcast.
  const int tsel = r16 & 3;
  const float xs = tsel == 0 ? umax[0] : tsel == 1 ? umax[1] : tsel == 2 ? umax[2] : umax[3];
  const float qx = 127.0f / xs;
  const float invx = (xs == 0.0f) ? 0.0f : qx;
  const float inv[4] = {quad_bcast<0>(invx), quad_bcast<1>(invx), quad_bcast<2>(invx),
                        quad_bcast<3>(invx)};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(u[t] * inv[t]), 0.0f, 127.0f);
    const uint32_t uc = static_cast<uint32_t>(r);
    stage[(t * 4 + grp) * 16 + pslot] = static_cast<uint8_t>(uc);
    if (DEBUG && a.dbg.pcode && grp < nh) {
      const int pos = PAGE * (j0 + t) + r16;
      if (t < np && pos < main_end) a.dbg.pcode[(qb + grp) * a.dbg.max_ctx + pos] = static_cast<uint8_t>(uc);
    }
  }
  // running reference max of each head; rescale what is accumulated when
  // some head's maximum moved (otherwise every factor would be exactly 1)
  const float Zn = fmaxf(st.Zr, fmaxf(fmaxf(zmax[0], zmax[1]), fmaxf(zmax[2], zmax[3])));
  if (__builtin_amdgcn_ballot_w64(Zn != st.Zr) != 0) {
    const float al = __builtin_amdgcn_exp2f(st.Zr - Zn);
#pragma unroll
    for (int o = 0; o < 8; ++o) st.O[o] *= al;
    st.Ls *= al;
    st.Ms *= al;
  }
  st.Zr = Zn;
  float wsu[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float wt = __builtin_amdgcn_exp2f(zmax[t] - Zn);
    st.Ls = __builtin_fmaf(wt, e[t], st.Ls);
    st.Ms = __builtin_fmaf(wt, emv[t], st.Ms);
    wsu[t] = wt * (umax[t] * (1.0f / 127.0f));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // A operand of PV: row 4h + tile, k-group = tile (block diagonal)
  v4i pa = *reinterpret_cast<const v4i*>(stage + (grp * 4 + (r16 >> 2)) * 16);
  if ((r16 & 3) != grp) pa = v4i{0, 0, 0, 0};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const v4i bv = e2 == 0 ? nib_positions(q.vq[s2].x, q.vq[s2].y) : nib_positions(q.vq[s2].z, q.vq[s2].w);
      const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa, bv, v4i{0, 0, 0, 0}, 0, 0, 0);
      // lane: head grp, channel 8 r16 + 2 s2 + e2, tile v in register v
      const int o = 2 * s2 + e2;
      float x = st.O[o];
      x = __builtin_fmaf(wsu[0], static_cast<float>(acc[0]), x);
      x = __builtin_fmaf(wsu[1], static_cast<float>(acc[1]), x);
      x = __builtin_fmaf(wsu[2], static_cast<float>(acc[2]), x);
      x = __builtin_fmaf(wsu[3], static_cast<float>(acc[3]), x);
      st.O[o] = x;
      if (DEBUG && a.dbg.pv && grp < nh) {
        const int ch = 8 * r16 + 2 * s2 + e2;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < np) a.dbg.pv[((qb + grp) * a.dbg.max_pages + (j0 + t)) * HD + ch] = acc[t];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------- page formats --
// The main kernel streams units of kUnit pages of one segment through its
// per-wave LDS slot; a format supplies the staging, the compute step, the
// order of the query operand and the partial it leaves.

// KV4-RL main region: quads of 4 INT4 pages (layouts above).
enum class QueryMode { Int8EvenOdd, Int8Natural, Bf16 };

struct Kv4Format {
  static constexpr QueryMode kQuery = QueryMode::Int8EvenOdd;
  static constexpr int kUnit = 4;
  static constexpr int kSlotBytes = kQuadSlotBytes;
  static constexpr int kWavesPerSimd = KV4_MAIN_WAVES_PER_SIMD;
  static constexpr int kBlock = BLOCK_BYTES;
  static constexpr bool kProtected = true;      // protected-region workgroups in the grid tail
  typedef QuadRegs Regs;
  typedef MainState State;
  __device__ static void to_lds(uint8_t* slot, const gptr* blk, int np, int lane, int r16, int grp) {
    quad_to_lds(slot, blk, np, lane, r16, grp);
  }
  __device__ static void from_lds(Regs& q, const uint8_t* slot, int lane, int r16, int grp) {
    (void)grp;
    quad_from_lds(q, slot, lane, r16);
  }
  // work done on a unit before the next unit's loads are issued into the slot: none
  __device__ static void before_issue(const DecArgs&, State&, Regs&, int, int, int, uint8_t*, int, int) {}
  __device__ static void reset(State& st, const uint8_t* slot, int r16, int grp) {
    (void)slot;
    (void)r16;
    (void)grp;
    st.Zr = -INFINITY;
    st.Ls = 0.0f;
    st.Ms = 0.0f;
#pragma unroll
    for (int o = 0; o < 8; ++o) st.O[o] = 0.0f;
  }
  template <bool DEBUG>
  __device__ static void compute(const DecArgs& a, State& st, const Regs& q, int np, v4i qa0, v4i qa1,
                                 float c_q, float S_q, int j0, int main_end, size_t qb, int nh, uint8_t* slot,
                                 int r16, int grp, int pslot) {
    compute_quad<DEBUG>(a, st, q, np, qa0, qa1, c_q, S_q, j0, main_end, qb, nh, slot + kSlotP, r16, grp,
                        pslot);
  }
  // A = O + sum(w e m_v); lane (head grp, r16) holds channels 8 r16 .. 8 r16 + 7 in A[0..7]
  __device__ static void finish(const State& st, float A[8], float& Z, float& L) {
    const float Mh = row16_sum(st.Ms);
    L = row16_sum(st.Ls);
    Z = st.Zr;
#pragma unroll
    for (int o = 0; o < 8; ++o) A[o] = st.O[o] + Mh;
  }
  // P0: the 4 heads' partials of the slot, kPart floats apart; this lane's head is grp
  __device__ static void store(float* P0, const float A[8], int r16, int grp) {
    float* P = P0 + grp * kPart + 8 * r16;  // 16-byte aligned: kPart * 4 = 528 = 16 * 33
    *reinterpret_cast<float4*>(P) = make_float4(A[0], A[1], A[2], A[3]);
    *reinterpret_cast<float4*>(P + 4) = make_float4(A[4], A[5], A[6], A[7]);
  }
};

// KV8 everywhere: pairs of 2 INT8 pages, every position through the protected
// path's arithmetic (INT8 QK on MFMA, FP32 softmax weights, v^ = bf16(s_v c),
// FP32 P times BF16 v^ with FP32 accumulation).  P enters the BF16 MFMA as the
// sum of two BF16 parts, hi = bf16(e) and lo = bf16(e - hi), which carries
// e to 16 significant bits (relative error below 2^-16).  PV on
// 16x16x32 MFMAs: MFMA r of accumulator acc keeps P only in rows 4r .. 4r+3
// (head = row % 4) and takes channels 64 acc + 16 r + n as its columns, so
// the four MFMAs fill all 16 rows of one accumulator with 4 heads x 64
// channels.  Slot layout:
//   [0, 4096)     K operands: page t, channel half h at 2048 t + 1024 h + 16 lane
//                 (lane (r16, grp): position r16, channels 64 h + 16 grp .. + 15)
//   [4096, 8192)  V codes, page t at 4096 + 2048 t (the block's channel-major copy)
//   [8192, 8320)  scales, page t at 8192 + 64 t: s_k[16], s_v[16]
//   [8320, 8832)  P operand [hi, lo][head][32 positions] BF16
constexpr int k8K = 0, k8V = 4096, k8S = 8192, k8P = 8320;
static_assert(k8P + 512 <= kSlotQ, "the KV8 slot must leave the query area free");

struct Kv8Regs {
  v4i kop[2][2];
  uint2 vq[8];
  uint32_t sk[2];
  uint4 sv;
};
// O[acc]: lane (r16, grp) holds head h (register h), channel 64 acc + 16 grp + r16
struct Kv8State {
  float Zr, Ls;
  v4f O[2];
};

template <bool DEBUG>
__device__ __forceinline__ void compute_pair(const DecArgs& a, Kv8State& st, const Kv8Regs& r, int np,
                                             v4i qa0, v4i qa1, float c_q, int j0, int L, size_t qb, int nh,
                                             uint8_t* slot, int r16, int grp) {
  // INT8 QK of the two pages; lane (head grp, position r16) after the move
  v4i d[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa0, r.kop[t][0], v4i{0, 0, 0, 0}, 0, 0, 0);
    d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa1, r.kop[t][1], d[t], 0, 0, 0);
  }
  float z[2];
  bool valid[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int D8 = qk_rows(d[t]);
    const int pos = PAGE * (j0 + t) + r16;
    valid[t] = (t < np) && (pos < L);
    z[t] = valid[t] ? (static_cast<float>(D8) * f16_value(r.sk[t])) * c_q : -INFINITY;
    if (DEBUG && valid[t] && a.dbg.qk && grp < nh) a.dbg.qk[(qb + grp) * a.dbg.max_ctx + pos] = D8;
  }
  // running max of each head; weights relative to it, earlier sums rescaled
  const float Zn = fmaxf(st.Zr, row16_max(fmaxf(z[0], z[1])));
  const bool moved = __builtin_amdgcn_ballot_w64(Zn != st.Zr) != 0;  // rescale needed
  const float al = __builtin_amdgcn_exp2f(st.Zr - Zn);
  st.Zr = Zn;
  float e[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) e[t] = valid[t] ? exp2s(z[t] - Zn) : 0.0f;
  st.Ls = __builtin_fmaf(st.Ls, al, e[0] + e[1]);
  // P operand through the slot: [hi, lo][head grp][16 t + r16]
  uint16_t* pst = reinterpret_cast<uint16_t*>(slot + k8P);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t hi = pack_bf16x2(e[t], 0.0f) & 0xFFFFu;
    const uint32_t lo = pack_bf16x2(e[t] - __uint_as_float(hi << 16), 0.0f) & 0xFFFFu;
    pst[grp * 32 + 16 * t + r16] = static_cast<uint16_t>(hi);
    pst[128 + grp * 32 + 16 * t + r16] = static_cast<uint16_t>(lo);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // A operand: lane (row r16, k-group grp) = head r16 % 4, positions 8 grp .. 8 grp + 7
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 ph = *reinterpret_cast<const u4*>(pst + (r16 & 3) * 32 + 8 * grp);
  const u4 pl = *reinterpret_cast<const u4*>(pst + 128 + (r16 & 3) * 32 + 8 * grp);
  // B operand: lane (r16, grp) = channel 16 s + r16, positions 8 (grp & 1) + i of
  // page grp >> 1; the V scale of a position outside the context is taken as 0
  const int tp = grp >> 1;
  const int pos0 = PAGE * (j0 + tp) + 8 * (grp & 1);
  // packed FP16 scales, positions outside the context zeroed
  uint32_t svw[4] = {r.sv.x, r.sv.y, r.sv.z, r.sv.w};
  const int nval = tp < np ? min(8, max(0, L - pos0)) : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t keep = (2 * i < nval ? 0x0000FFFFu : 0u) | (2 * i + 1 < nval ? 0xFFFF0000u : 0u);
    svw[i] &= keep;
  }
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  // rescale what is accumulated (head h in register h) when some head's
  // maximum moved; otherwise every factor is exactly 1
  if (moved) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float alh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 16 * h));
      st.O[0][h] *= alh;
      st.O[1][h] *= alh;
    }
  }
  const u4 zero4 = u4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < 8; ++s) {  // channel block s = 4 acc + r
    // v^ = bf16(s_v c); s_v c is exact in FP32 (an FMA with zero addend
    // taking the FP16 scale directly)
    const uint32_t w0 = r.vq[s].x, w1 = r.vq[s].y;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const h2 sp = __builtin_bit_cast(h2, svw[i >> 1]);
      const float si = static_cast<float>(sp[i & 1]);
      const float c = static_cast<float>(static_cast<int8_t>((i < 4 ? w0 : w1) >> (8 * (i & 3))));
      x[i] = __builtin_fmaf(si, c, 0.0f);
    }
    const u4 pk = u4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    const v8bf vb = __builtin_bit_cast(v8bf, pk);
    const bool mine = (r16 >> 2) == (s & 3);  // rows 4r .. 4r+3 carry P in MFMA r
    const v8bf ah = __builtin_bit_cast(v8bf, mine ? ph : zero4);
    const v8bf alo = __builtin_bit_cast(v8bf, mine ? pl : zero4);
    v4f o = st.O[s >> 2];
    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vb, o, 0, 0, 0);
    st.O[s >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, vb, o, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep one block's operands live at a time
  }
  __builtin_amdgcn_wave_barrier();
}

struct Kv8Format {
  static constexpr QueryMode kQuery = QueryMode::Int8Natural;
  static constexpr int kUnit = 2;
  static constexpr int kSlotBytes = kQuadSlotBytes;
  static constexpr int kWavesPerSimd = KV8_MAIN_WAVES_PER_SIMD;
  static constexpr int kBlock = KV8_BLOCK_BYTES;
  static constexpr bool kProtected = false;
  typedef Kv8Regs Regs;
  typedef Kv8State State;
  // every tile is loaded (past the piece's last page: that page again)
  __device__ static void to_lds(uint8_t* slot, const gptr* blk, int np, int lane, int r16, int grp) {
    (void)np;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_global_load_lds(blk[t] + HD * r16 + 64 * h + 16 * grp,
                                         (lptr)(slot + k8K + 2048 * t + 1024 * h), 16, 0, kNT);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(blk[t] + KV8_OFF_V + 1024 * i + 16 * lane,
                                         (lptr)(slot + k8V + 2048 * t + 1024 * i), 16, 0, kNT);
    if (lane < 8)  // 2 pages x 64 B of scales
      __builtin_amdgcn_global_load_lds((lane < 4 ? blk[0] : blk[1]) + KV8_OFF_SK + 16 * (lane & 3),
                                       (lptr)(slot + k8S), 16, 0, kNT);
  }
  __device__ static void from_lds(Regs& r, const uint8_t* slot, int lane, int r16, int grp) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        r.kop[t][h] = *reinterpret_cast<const v4i*>(slot + k8K + 2048 * t + 1024 * h + 16 * lane);
    const uint8_t* vb = slot + k8V + 2048 * (grp >> 1) + 16 * r16 + 8 * (grp & 1);
#pragma unroll
    for (int s = 0; s < 8; ++s) r.vq[s] = *reinterpret_cast<const uint2*>(vb + 256 * s);
#pragma unroll
    for (int t = 0; t < 2; ++t) r.sk[t] = *reinterpret_cast<const uint16_t*>(slot + k8S + 64 * t + 2 * r16);
    r.sv = *reinterpret_cast<const uint4*>(slot + k8S + 64 * (grp >> 1) + 32 + 16 * (grp & 1));
  }
  __device__ static void before_issue(const DecArgs&, State&, Regs&, int, int, int, uint8_t*, int, int) {}
  __device__ static void reset(State& st, const uint8_t* slot, int r16, int grp) {
    (void)slot;
    (void)r16;
    (void)grp;
    st.Zr = -INFINITY;
    st.Ls = 0.0f;
    st.O[0] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    st.O[1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  template <bool DEBUG>
  __device__ static void compute(const DecArgs& a, State& st, const Regs& r, int np, v4i qa0, v4i qa1,
                                 float c_q, float S_q, int j0, int main_end, size_t qb, int nh, uint8_t* slot,
                                 int r16, int grp, int pslot) {
    (void)S_q;
    (void)pslot;
    compute_pair<DEBUG>(a, st, r, np, qa0, qa1, c_q, j0, main_end, qb, nh, slot, r16, grp);
  }
  // A[4 acc + h]: head h, channel 64 acc + 16 grp + r16
  __device__ static void finish(const State& st, float A[8], float& Z, float& L) {
    L = row16_sum(st.Ls);
    Z = st.Zr;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      A[h] = st.O[0][h];
      A[4 + h] = st.O[1][h];
    }
  }
  // P0: the 4 heads' partials of the slot, kPart floats apart
  __device__ static void store(float* P0, const float A[8], int r16, int grp) {
#pragma unroll
    for (int acc = 0; acc < 2; ++acc)
#pragma unroll
      for (int h = 0; h < 4; ++h) P0[h * kPart + 64 * acc + 16 * grp + r16] = A[4 * acc + h];
  }
};

// MXFP4 variant of the main region (KV4-RL pages, comparison of 4-bit formats,
// appendix D.4): units of 4 pages in OCP MXFP4, attended on their exactly
// dequantized values.  QK: the BF16-rounded rotated query against K codes
// converted to BF16 by the hardware FP4 conversion with the block's E8M0 scale
// (v_cvt_scalef32_pk_bf16_fp4), BF16 MFMA 16x16x32 with FP32 accumulation.
// The four MFMAs of a tile take the channels in a relabelled order that is the
// same for both operands: MFMA m, lane group grp covers channels
// 32 grp + 8 m .. + 7, so a lane's operands of all four come from its own
// 16 bytes of the position's K codes (one LDS read) and one block scale; the
// query operands follow the same order and are read once per piece.  PV: the FP32 weight of a position
// times 2^(V block exponent) is split into two BF16 parts per V block and
// meets the unscaled V codes (converted at unit scale) on the same MFMA, rows
// rotated as for KV8; the P operands of one V block at a time pass through
// the slot (double buffered), which keeps the slot at 9728 B.  A unit is two
// pairs: the first is computed before the next unit's loads are issued, then
// the second pair's codes are read into registers, the loads go out, and the
// second pair is computed while they stream.  Slot layout:
//   [0, 4096)     K codes in operand order, page t at 1024 t: lane (r16, c)
//                 holds channel block c of position r16 at 16 (r16 + 16 c)
//   [4096, 8192)  V codes, page t at 4096 + 1024 t (the block's channel-major copy)
//   [8192, 8704)  scales, page t at 8192 + 128 t: K E8M0 [16][4], V E8M0 [16][4]
//   [8704, 9728)  the BF16 rotated query [head][128] when a piece starts (read
//                 into registers), then P operands of V block b at
//                 8704 + 512 (b & 1): [hi, lo][head][32 positions] BF16
//   [9728, 9744)  16 zero bytes: the A operand of the lanes whose rows carry
//                 no P in an MFMA is read from here (no selects)
constexpr int kmxK = 0, kmxV = 4096, kmxS = 8192, kmxQ = 8704, kmxP = 8704, kmxZ = 9728, kmxSlotBytes = 9744;

struct MxState {
  Kv8State s;
  v8bf qa[4];  // A operands of QK: row r16 = head r16 / 4, channels 32 grp + 8 m .. + 7
};

struct MxRegs {  // one pair of pages
  uint4 k[2];        // page t, channel block grp of position r16: component m = channels 32 grp + 8 m .. + 7
  uint32_t ks[2], vs[2];
  uint32_t vq[8];    // 8 FP4 codes: positions 8 (grp & 1) .. of channel 16 s + r16, page grp >> 1 of the pair
};

__device__ __forceinline__ float e8m0_value(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);  // 2^(e - 127); e = 0 is the subnormal 2^-127
}

// 8 FP4 codes (4 bytes, low nibble first) times scale, as 8 BF16.
__device__ __forceinline__ v8bf fp4x8_bf16(uint32_t w, float scale) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const b2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const b2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const b2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One pair of pages (np of them in the region, the first at logical page j0).
__device__ __forceinline__ void compute_mx_pair(const DecArgs& a, MxState& ms, const MxRegs& r, int np,
                                                int j0, int main_end, uint8_t* slot, int r16, int grp) {
  Kv8State& st = ms.s;
  // QK on BF16 MFMAs; lane (head grp, position r16) after the move
  float z[2];
  bool valid[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float sc = e8m0_value((r.ks[t] >> (8 * grp)) & 0xFFu);  // this lane's K block
    const uint32_t kw[4] = {r.k[t].x, r.k[t].y, r.k[t].z, r.k[t].w};
    v4f d = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ms.qa[m], fp4x8_bf16(kw[m], sc), d, 0, 0, 0);
    const float D = d[0];  // rows 4 grp .. 4 grp + 3 all hold head grp
    const int pos = PAGE * (j0 + t) + r16;
    valid[t] = (t < np) && (pos < main_end);
    z[t] = valid[t] ? D * a.scale_log2 : -INFINITY;
  }
  const float Zn = fmaxf(st.Zr, row16_max(fmaxf(z[0], z[1])));
  // what is accumulated is rescaled only when some head's maximum moved
  // (otherwise every factor is exactly 1)
  const bool moved = __builtin_amdgcn_ballot_w64(Zn != st.Zr) != 0;
  const float al = __builtin_amdgcn_exp2f(st.Zr - Zn);
  st.Zr = Zn;
  float e[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) e[t] = valid[t] ? exp2s(z[t] - Zn) : 0.0f;
  st.Ls = __builtin_fmaf(st.Ls, al, e[0] + e[1]);
  if (moved) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float alh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 16 * h));
      st.O[0][h] *= alh;
      st.O[1][h] *= alh;
    }
  }
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const uint8_t* zrow = slot + kmxZ;
  // the weight as two BF16 parts, hi = bf16(e) and lo = bf16(e - hi), kept
  // as FP32 values whose low 16 bits are zero
  float ehi[2], elo[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ehi[t] = __uint_as_float(pack_bf16x2(0.0f, e[t]) & 0xFFFF0000u);
    elo[t] = __uint_as_float(pack_bf16x2(0.0f, e[t] - ehi[t]) & 0xFFFF0000u);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // P operand of V block b: both parts times 2^(E_v(b) - 127), a power of
    // two, so each stays a BF16 value (its high 16 bits are stored)
    uint16_t* pst = reinterpret_cast<uint16_t*>(slot + kmxP + 512 * (b & 1));  // [hi, lo][head][32]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ex = static_cast<int>((r.vs[t] >> (8 * b)) & 0xFFu) - 127;
      pst[grp * 32 + 16 * t + r16] = static_cast<uint16_t>(__float_as_uint(__builtin_ldexpf(ehi[t], ex)) >> 16);
      pst[(4 + grp) * 32 + 16 * t + r16] = static_cast<uint16_t>(__float_as_uint(__builtin_ldexpf(elo[t], ex)) >> 16);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // A operand: head r16 % 4, positions 8 grp .. 8 grp + 7, in the rows of
    // MFMA r only (r = sv % 4), zero elsewhere
    const uint8_t* hrow = reinterpret_cast<const uint8_t*>(pst + (r16 & 3) * 32 + 8 * grp);
    const uint8_t* lrow = reinterpret_cast<const uint8_t*>(pst + (4 + (r16 & 3)) * 32 + 8 * grp);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int sv = 2 * b + half;  // channels 16 sv .. 16 sv + 15 = 4 acc + r
      const v8bf vb = fp4x8_bf16(r.vq[sv], 1.0f);
      const bool mine = (r16 >> 2) == (sv & 3);
      const u4 ph = *reinterpret_cast<const u4*>(mine ? hrow : zrow);
      const u4 pl = *reinterpret_cast<const u4*>(mine ? lrow : zrow);
      v4f o = st.O[sv >> 2];
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ph), vb, o, 0, 0, 0);
      st.O[sv >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, pl), vb, o, 0, 0, 0);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

struct MxFormat {
  static constexpr QueryMode kQuery = QueryMode::Bf16;
  static constexpr int kUnit = 4;
  static constexpr int kSlotBytes = kmxSlotBytes;
  static constexpr int kWavesPerSimd = KV4_MAIN_WAVES_PER_SIMD;
  static constexpr int kBlock = BLOCK_BYTES;
  static constexpr bool kProtected = true;
  typedef MxRegs Regs;
  typedef MxState State;
  // every tile is loaded (past the piece's last page: that page again)
  __device__ static void to_lds(uint8_t* slot, const gptr* blk, int np, int lane, int r16, int grp) {
    (void)np;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_global_load_lds(blk[t] + 64 * r16 + 16 * grp, (lptr)(slot + kmxK + 1024 * t), 16, 0, kNT);
      __builtin_amdgcn_global_load_lds(blk[t] + OFF_VCODE + 16 * lane, (lptr)(slot + kmxV + 1024 * t), 16, 0, kNT);
    }
    if (lane < 32)  // 4 pages x 128 B of scales
      __builtin_amdgcn_global_load_lds(blk[lane >> 3] + OFF_KMETA + 16 * (lane & 7), (lptr)(slot + kmxS), 16, 0, kNT);
  }
  // the codes and scales of pair p (pages 2p, 2p + 1 of the unit)
  __device__ static void pair_from_lds(Regs& r, const uint8_t* slot, int p, int r16, int grp) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pg = 2 * p + t;
      r.k[t] = *reinterpret_cast<const uint4*>(slot + kmxK + 1024 * pg + 16 * (r16 + 16 * grp));
      r.ks[t] = *reinterpret_cast<const uint32_t*>(slot + kmxS + 128 * pg + 4 * r16);
      r.vs[t] = *reinterpret_cast<const uint32_t*>(slot + kmxS + 128 * pg + 64 + 4 * r16);
    }
    const uint8_t* vb = slot + kmxV + 1024 * (2 * p + (grp >> 1)) + 8 * r16 + 4 * (grp & 1);
#pragma unroll
    for (int sv = 0; sv < 8; ++sv) r.vq[sv] = *reinterpret_cast<const uint32_t*>(vb + 128 * sv);
  }
  __device__ static void from_lds(Regs& r, const uint8_t* slot, int lane, int r16, int grp) {
    (void)lane;
    pair_from_lds(r, slot, 0, r16, grp);
  }
  // the unit's first pair, then the second pair's codes into registers (the
  // slot is then free for the next unit's loads)
  __device__ static void before_issue(const DecArgs& a, State& st, Regs& r, int np, int j0, int main_end,
                                      uint8_t* slot, int r16, int grp) {
    compute_mx_pair(a, st, r, min(np, 2), j0, main_end, slot, r16, grp);
    if (np > 2) pair_from_lds(r, slot, 1, r16, grp);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }
  // a new piece: fresh state, and the query operands from the slot's query area
  __device__ static void reset(State& st, uint8_t* slot, int r16, int grp) {
    Kv8Format::reset(st.s, slot, r16, grp);
    if (r16 == 0 && grp == 0) *reinterpret_cast<uint4*>(slot + kmxZ) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      st.qa[m] = *reinterpret_cast<const v8bf*>(slot + kmxQ + 2 * (HD * (r16 >> 2) + 32 * grp + 8 * m));
  }
  template <bool DEBUG>
  __device__ static void compute(const DecArgs& a, State& st, const Regs& r, int np, v4i qa0, v4i qa1,
                                 float c_q, float S_q, int j0, int main_end, size_t qb, int nh, uint8_t* slot,
                                 int r16, int grp, int pslot) {
    (void)nh;
    (void)qa0;
    (void)qa1;
    (void)c_q;
    (void)S_q;
    (void)pslot;
    (void)qb;
    if (np > 2) compute_mx_pair(a, st, r, np - 2, j0 + 2, main_end, slot, r16, grp);
  }
  __device__ static void finish(const State& st, float A[8], float& Z, float& L) { Kv8Format::finish(st.s, A, Z, L); }
  __device__ static void store(float* P0, const float A[8], int r16, int grp) { Kv8Format::store(P0, A, r16, grp); }
};

// Work split of the main region: the global page list (sequence-major, then
// query-head group, then logical page; T pages; a kv-head with more than 4
// query heads has its pages listed once per group) is cut into one contiguous chunk per
// wave, chunk c = [floor(T c / nw), floor(T (c+1) / nw)) when T >= nw (no
// chunk empty), else [min(c, T), min(c+1, T)) (empty chunks only at the end).
// A wave writes one partial per segment its chunk touches, at slot
// c + b*Hv + v: chunks visit segments in list order, so slots never collide
// and nw + B*Hv slots suffice.  The waves holding a segment's first and last
// pages record their chunk indices for the merge, which reads every chunk in
// between: none of them may be empty.
// floor(T c / nw) is evaluated in 32 bits as q c + floor(r c / nw) with
// T = q nw + r (r c < nw^2 <= 2^32 for the at most 65536 waves of a grid),
// two 32-bit divisions in place of a 64-bit one.
struct Split {
  int T, nw;
  uint32_t q, r;
};
__device__ __forceinline__ Split make_split(int T, int nw) {
  const uint32_t q = static_cast<uint32_t>(T) / static_cast<uint32_t>(nw);
  return Split{T, nw, q, static_cast<uint32_t>(T) - q * static_cast<uint32_t>(nw)};
}
__device__ __forceinline__ int chunk_begin(const Split& s, int c) {  // wave-uniform, scalar
  const uint32_t uc = static_cast<uint32_t>(c);
  return s.T >= s.nw ? static_cast<int>(s.q * uc + (s.r * uc) / static_cast<uint32_t>(s.nw)) : min(c, s.T);
}

// The plan as seen by one main-kernel wave.  For up to 256 sequences every
// wave builds it in registers from the context lengths (entry i, 1 <= i <= B,
// in lane (i-1) / 4 of register (i-1) % 4): one round of loads and a wave
// prefix sum, then lookups are readlanes and ballots.  Larger batches read
// the plan a separate launch wrote, through scalar loads.
struct PlanView {
  const int32_t* plan;
  int B, T;
  bool in_regs;
  int v[4];
};
__device__ __forceinline__ PlanView plan_view(const DecArgs& a, int lane) {
  PlanView r;
  r.plan = a.ws.plan;
  r.B = a.B;
  r.in_regs = a.B <= 256;
  if (!r.in_regs) {
    r.T = ld_const(a.ws.plan + a.B);
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = 0;
    return r;
  }
  // the four context lengths of the lane, loaded together (the empty asm
  // statement keeps the compiler from moving each load into the branch that
  // uses it, which made them four dependent round trips)
  int Lv[4], m[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) Lv[k] = a.ctx[min(4 * lane + k, a.B - 1)];
  asm volatile("" : "+v"(Lv[0]), "+v"(Lv[1]), "+v"(Lv[2]), "+v"(Lv[3]));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int mp = main_pages(Lv[k], Lv[k], a.sink, a.window) * a.Hv;
    m[k] = 4 * lane + k < a.B ? mp : 0;
  }
  m[1] += m[0];
  m[2] += m[1];
  m[3] += m[2];
  const int x = wave_incl_sum_i(m[3], lane);  // inclusive prefix of the lane totals
  const int excl = x - m[3];
#pragma unroll
  for (int k = 0; k < 4; ++k) r.v[k] = excl + m[k];
  r.T = __builtin_amdgcn_readlane(r.v[3], 63);
  return r;
}
// plan[i] for a wave-uniform 0 <= i <= B.
__device__ __forceinline__ int plan_at(const PlanView& r, int i) {
  if (!r.in_regs) return ld_const(r.plan + i);
  if (i == 0) return 0;
  const int l = (i - 1) >> 2, k = (i - 1) & 3;
  const int x0 = __builtin_amdgcn_readlane(r.v[0], l), x1 = __builtin_amdgcn_readlane(r.v[1], l);
  const int x2 = __builtin_amdgcn_readlane(r.v[2], l), x3 = __builtin_amdgcn_readlane(r.v[3], l);
  return k == 0 ? x0 : k == 1 ? x1 : k == 2 ? x2 : x3;
}
// Sequence b holding page p (plan[b] <= p < plan[b+1]), at or after lo.
__device__ __forceinline__ int find_seq(const PlanView& r, int p, int lo, int lane) {
  if (r.in_regs) {  // count the entries 1..B that are <= p
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      cnt += __builtin_popcountll(__ballot(4 * lane + k + 1 <= r.B && r.v[k] <= p));
    return cnt;
  }
  int hi = r.B;  // plan[lo] <= p < plan[hi]; scalar loads, counted apart from vector loads
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_const(r.plan + mid) <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One quad of the wave's page stream.
struct PageIds {  // physical pages of a unit's tiles (wave-uniform)
  int id[4];
};

struct QuadDesc {
  int b, g, j0, np, slot, main_end;
  int gp, h0;          // the group's kv-head and first query head
  bool first, last;    // first / last quad of its piece
  bool opens, closes;  // the piece starts at the segment's first page / ends at its last
};

template <class F, bool DEBUG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(F::kWavesPerSimd, F::kWavesPerSimd))) void main_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][F::kSlotBytes];
  static_assert(kProtLdsFused <= 4 * F::kSlotBytes, "the protected role reuses the main role's LDS");
  const int nw = a.ws.n_waves;
  if constexpr (F::kProtected) {
    if (blockIdx.x >= nw / 4) {  // protected-region workgroups fill the tail of the grid
      const int u = blockIdx.x - nw / 4;
      protected_partial<DEBUG>(a, u % a.Hv, u / a.Hv, &lds[0][0]);
      return;
    }
  }
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * 4 + wave;
  const PlanView pv = plan_view(a, lane);
  const Split sp = make_split(pv.T, nw);
  uint8_t* slot = lds[wave];
  const int pslot = pcode_slot(r16);
  const size_t pstride = static_cast<size_t>(a.Hkv) * F::kBlock;

  // ---- issue cursor: page ip of the chunk [ip, iend) and the segment holding it
  int ip = chunk_begin(sp, w);
  const int iend = chunk_begin(sp, w + 1);
  const int chunk0 = ip;
  int ib = ip < iend ? find_seq(pv, ip, 0, lane) : 0;
  int seg0 = 0, seg_end = 0, seg_g = 0;  // segment holding ip: pages [seg0, seg_end), head group seg_g
  HeadGroup seg_hg{0, 0, 1};               // seg_g's kv-head and query heads
  // Q operands of the next piece: the raw query is loaded when its first quad
  // is described (raw2, moved to raw1 with the quad), and rotated/quantized
  // after the compute of the iteration that issued that quad.
  v4i nqa0 = {0, 0, 0, 0}, nqa1 = {0, 0, 0, 0};
  float2 nqi = make_float2(0.0f, 0.0f);
  uint4 raw1 = make_uint4(0, 0, 0, 0), raw2 = make_uint4(0, 0, 0, 0);
  auto group_query = [&](const QuadDesc& d, const uint4& raw) {
    if constexpr (F::kQuery == QueryMode::Bf16) {
      // the rotated query rounded to BF16, natural order: head grp, channels 8 r16 ..
      (void)d;
      float x[8];
      rotate_group_query(raw, r16, x);
      const uint4 w = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                                 pack_bf16x2(x[6], x[7]));
      *reinterpret_cast<uint4*>(slot + kmxQ + 2 * (HD * grp + 8 * r16)) = w;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      return;
    }
    const GroupQuery gq = quantize_group_query(raw, a.scale_log2, r16);
    if (DEBUG) {  // lane (grp, r16) holds rotated channels 8 r16 .. 8 r16 + 7 (same values from every piece)
      const size_t bh = static_cast<size_t>(d.b) * a.Hq + d.h0 + grp;
      if (grp < min(4, (d.gp + 1) * a.G - d.h0) && a.dbg.qcodes)
#pragma unroll
        for (int j = 0; j < 8; ++j) a.dbg.qcodes[bh * HD + 8 * r16 + j] = static_cast<int8_t>(gq.c[j]);
      if (grp < min(4, (d.gp + 1) * a.G - d.h0) && a.dbg.qsum && r16 == 0) a.dbg.qsum[bh] = gq.S;
    }
    // A operand of QK: row r = head r / 4, k = channels (lane group grp
    // covers channels 32grp..32grp+31, even / odd split); the codes go
    // through the slot's query area to reach that layout.
    uint8_t* qs = slot + kSlotQ + grp * HD;
    if constexpr (F::kQuery == QueryMode::Int8Natural) {  // channels 8 r16 .. 8 r16 + 7 in place
      const uint32_t lo = (gq.c[0] & 0xFF) | ((gq.c[1] & 0xFF) << 8) | ((gq.c[2] & 0xFF) << 16) |
                          (static_cast<uint32_t>(gq.c[3] & 0xFF) << 24);
      const uint32_t hi = (gq.c[4] & 0xFF) | ((gq.c[5] & 0xFF) << 8) | ((gq.c[6] & 0xFF) << 16) |
                          (static_cast<uint32_t>(gq.c[7] & 0xFF) << 24);
      reinterpret_cast<uint2*>(qs)[r16] = make_uint2(lo, hi);
    } else {
      const uint32_t even = (gq.c[0] & 0xFF) | ((gq.c[2] & 0xFF) << 8) | ((gq.c[4] & 0xFF) << 16) |
                            (static_cast<uint32_t>(gq.c[6] & 0xFF) << 24);
      const uint32_t odd = (gq.c[1] & 0xFF) | ((gq.c[3] & 0xFF) << 8) | ((gq.c[5] & 0xFF) << 16) |
                           (static_cast<uint32_t>(gq.c[7] & 0xFF) << 24);
      reinterpret_cast<uint32_t*>(qs)[r16] = even;
      reinterpret_cast<uint32_t*>(qs + 64)[r16] = odd;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // A operand of QK: row r16 = head r16 / 4 (qk_rows)
    nqa0 = *reinterpret_cast<const v4i*>(slot + kSlotQ + (r16 >> 2) * HD + 16 * grp);
    nqa1 = *reinterpret_cast<const v4i*>(slot + kSlotQ + (r16 >> 2) * HD + 64 + 16 * grp);
    nqi = make_float2(gq.c_q, __int_as_float(gq.S));
  };

  // Stage 1: describe the next quad of the chunk and fetch its page-table
  // entries (scalar loads, so that they do not count with the page loads in
  // vmcnt) into pt; false when the chunk is done.  Runs two quads ahead of the
  // compute.
  auto plan_quad = [&](QuadDesc& d, PageIds& pt) -> bool {
    if (ip >= iend) return false;
    if (ip >= seg_end || ip == chunk0) {  // entering a segment: locate it once
      while (plan_at(pv, ib + 1) <= ip) ++ib;
      const int pb = plan_at(pv, ib);
      const int mp = (plan_at(pv, ib + 1) - pb) / a.Hv;
      seg_g = (ip - pb) / mp;
      seg0 = pb + seg_g * mp;
      seg_end = seg0 + mp;
      seg_hg = head_group(a, seg_g);
    }
    const int stop = min(iend, seg_end);
    d.b = ib;
    d.g = seg_g;
    d.gp = seg_hg.gp;
    d.h0 = seg_hg.h0;
    d.j0 = a.sink / PAGE + (ip - seg0);
    d.np = min(F::kUnit, stop - ip);
    d.slot = w + ib * a.Hv + seg_g;
    d.first = (ip == chunk0) || (ip == seg0);
    d.last = ip + d.np >= stop;
    d.opens = ip == seg0;
    d.closes = stop == seg_end;
    const int32_t* ptrow = a.page_table + static_cast<size_t>(ib) * a.pt_stride;
#pragma unroll
    for (int t = 0; t < F::kUnit; ++t) pt.id[t] = ld_const(ptrow + d.j0 + min(t, d.np - 1));
    if (d.first)  // BF16 query of head grp, channels 8 r16 .. 8 r16 + 7
      // (a 32-bit byte offset from the query array's base, so that the base
      // stays in scalar registers: a 64-bit per-lane pointer held across the
      // loop was spilled in the MXFP4 instantiation and its reload waited for
      // every load in flight)
      raw2 = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint8_t*>(a.q) +
          (static_cast<uint32_t>(ib * a.Hq + seg_hg.h0 + min(grp, seg_hg.nh - 1)) * (2u * HD) + 16u * r16));
    ip += d.np;
    return true;
  };
  // Stage 2: start the page loads of a described quad into the LDS slot.
  auto issue_quad = [&](QuadDesc& d, const PageIds& pt) {
    const gptr gbase = (gptr)a.pages + static_cast<size_t>(d.gp) * F::kBlock;
    gptr blk[F::kUnit];
#pragma unroll
    for (int t = 0; t < F::kUnit; ++t)
      blk[t] = gbase + static_cast<size_t>(static_cast<uint32_t>(pt.id[t])) * pstride;
    F::to_lds(slot, blk, d.np, lane, r16, grp);
    if (d.first) {
      const int L = ld_const(a.ctx + d.b);
      d.main_end = main_end_of(L, L, a.window);
    }
  };

  // Pipeline: quad i is computed while quad i+1 streams into the LDS slot
  // and the page-table entries of quad i+2 are fetched; pieces and ranges
  // follow one another without a gap.
  QuadDesc d1, d2;  // quads i+1 (in flight) and i+2 (described)
  PageIds pt1{}, pt2{};
  bool have1 = plan_quad(d1, pt1);
  raw1 = raw2;
  if (have1) {
    issue_quad(d1, pt1);
    group_query(d1, raw1);  // d1 is the first quad of a piece
  }
  bool have2 = have1 && plan_quad(d2, pt2);
  typename F::State st;
  v4i qa0 = {0, 0, 0, 0}, qa1 = {0, 0, 0, 0};
  float c_q = 0.0f, S_q = 0.0f;
  int main_end = 0;
  // A finished piece's partial is held in registers and stored only when the
  // next piece finishes or the wave ends: stores count in the same vmcnt as
  // the page loads and complete slowly under the read stream, so a wave with
  // two pieces (the common case) never waits for one.
  bool pend = false;
  float* pend_P = nullptr;
  float pend_A[8], pend_Z = 0.0f, pend_L = 0.0f;
  int pend_bg = 0;
  bool pend_opens = false, pend_closes = false, piece_opens = false;
  auto store_partial = [&]() {
    F::store(pend_P, pend_A, r16, grp);
    if (r16 == 0) {
      pend_P[grp * kPart + 128] = pend_Z;
      pend_P[grp * kPart + 129] = pend_L;
    }
    // the chunks holding the segment's first and last pages bound its partials
    if (lane == 0 && pend_opens) a.ws.mrange[pend_bg].x = w;
    if (lane == 0 && pend_closes) a.ws.mrange[pend_bg].y = w;
  };
  while (have1) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    typename F::Regs q;
    F::from_lds(q, slot, lane, r16, grp);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const QuadDesc cd = d1;
    if (cd.first) {
      piece_opens = cd.opens;
      qa0 = nqa0;
      qa1 = nqa1;
      c_q = nqi.x;
      S_q = static_cast<float>(__float_as_int(nqi.y));
      main_end = cd.main_end;
      F::reset(st, slot, r16, grp);
    }
    F::before_issue(a, st, q, cd.np, cd.j0, main_end, slot, r16, grp);
    have1 = have2;
    if (have2) {
      d1 = d2;
      pt1 = pt2;
      raw1 = raw2;
      issue_quad(d1, pt1);
      have2 = plan_quad(d2, pt2);
    }
    const size_t qb = static_cast<size_t>(cd.b) * a.Hq + cd.h0;
    const int nh = min(4, (cd.gp + 1) * a.G - cd.h0);
    F::template compute<DEBUG>(a, st, q, cd.np, qa0, qa1, c_q, S_q, cd.j0, main_end, qb, nh, slot, r16,
                               grp, pslot);
    if (cd.last) {  // partial of the piece
      if (pend) store_partial();
      F::finish(st, pend_A, pend_Z, pend_L);
      pend_P = a.ws.parts + static_cast<size_t>(cd.slot) * GQA * kPart;
      pend_bg = cd.b * a.Hv + cd.g;
      pend_opens = piece_opens;
      pend_closes = cd.closes;
      pend = true;
    }
    if (have1 && d1.first) group_query(d1, raw1);  // operands for the next iteration
  }
  if (pend) store_partial();
}

// Exact log-sum-exp merge of the protected partial (none when s = w = 0) and
// the main partials of each head, one workgroup per (query-head group v,
// sequence b), wave h for the group's head h, lane l for channels 2l, 2l+1.
// Writes out and lse.
__global__ __launch_bounds__(256) void merge_kernel(DecArgs a) {
  const int g = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.Hv));
  const int b = static_cast<int>(blockIdx.x / static_cast<unsigned>(a.Hv));
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const HeadGroup hg = head_group(a, g);
  if (wave >= hg.nh) return;  // a row past the group's heads (no barrier below)
  const size_t bh = static_cast<size_t>(b) * a.Hq + hg.h0 + wave;
  float2 Am = make_float2(0.0f, 0.0f);
  float Zm = -INFINITY, lm = 0.0f;
  if (a.sink + a.window > 0) {
    const float* Pp = a.ws.prot + bh * kPart;
    Am = reinterpret_cast<const float2*>(Pp)[lane];
    Zm = Pp[128];
    lm = Pp[129];
  }
  // main partials: chunks c_lo..c_hi (recorded by the main kernel) at slots c + b*Hv + g
  const int bg = b * a.Hv + g;
  const int2 cr = a.ws.mrange[bg];  // written by the main kernel when the segment has pages
  const int Lb = ld_const(a.ctx + b);
  const int c_lo = cr.x, n_parts = main_pages(Lb, Lb, a.sink, a.window) > 0 ? cr.y - cr.x + 1 : 0;
  constexpr int kBatch = 4;
  for (int k0 = 0; k0 < n_parts; k0 += kBatch) {
    // loads of the batch first, all of them (indices past the last partial
    // repeat it and are skipped below), held together by the empty asm
    // statement so that they form one round trip
    float2 Ac[kBatch], Zl[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c_lo + min(k0 + i, n_parts - 1);
      const float* Pc = a.ws.parts + ((static_cast<size_t>(c) + bg) * GQA + wave) * kPart;
      Ac[i] = reinterpret_cast<const float2*>(Pc)[lane];
      Zl[i] = *reinterpret_cast<const float2*>(Pc + 128);  // Z, l
    }
    asm volatile("" : "+v"(Ac[0].x), "+v"(Ac[0].y), "+v"(Ac[1].x), "+v"(Ac[1].y), "+v"(Ac[2].x), "+v"(Ac[2].y),
                 "+v"(Ac[3].x), "+v"(Ac[3].y), "+v"(Zl[0].x), "+v"(Zl[0].y), "+v"(Zl[1].x), "+v"(Zl[1].y),
                 "+v"(Zl[2].x), "+v"(Zl[2].y), "+v"(Zl[3].x), "+v"(Zl[3].y));
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (k0 + i >= n_parts || Zl[i].x == -INFINITY) continue;
      const float Zn = fmaxf(Zm, Zl[i].x);
      const float w0 = __builtin_amdgcn_exp2f(Zm - Zn), w1 = __builtin_amdgcn_exp2f(Zl[i].x - Zn);
      Am.x = Am.x * w0 + Ac[i].x * w1;
      Am.y = Am.y * w0 + Ac[i].y * w1;
      lm = lm * w0 + Zl[i].y * w1;
      Zm = Zn;
    }
  }
  reinterpret_cast<float2*>(a.out + bh * HD)[lane] = make_float2(Am.x / lm, Am.y / lm);
  if (lane == 0) a.lse[bh] = 0.69314718055994531f * (Zm + log2f(lm));
}


}  // namespace

// Partial slots of the main region: chunk c writes segment (b, v) at c + b*Hv + v.
static size_t part_slots(int B, int Hv, int n_waves) {
  return static_cast<size_t>(n_waves) + static_cast<size_t>(B) * Hv;
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int n_waves) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const int Hv = query_head_groups(Hq, Hkv);
  size_t n = up(static_cast<size_t>(B + 1) * 4);
  n += up(static_cast<size_t>(B) * Hq * kPart * 4);
  n += up(static_cast<size_t>(B) * Hv * 8);
  n += up(part_slots(B, Hv, n_waves) * GQA * kPart * 4);
  return n;
}

DecodeWorkspace carve_workspace(void* base, int B, int Hq, int Hkv, int n_waves) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const int Hv = query_head_groups(Hq, Hkv);
  char* p = static_cast<char*>(base);
  DecodeWorkspace w;
  w.plan = reinterpret_cast<int32_t*>(p);
  p += up(static_cast<size_t>(B + 1) * 4);
  w.prot = reinterpret_cast<float*>(p);
  p += up(static_cast<size_t>(B) * Hq * kPart * 4);
  w.mrange = reinterpret_cast<int2*>(p);
  p += up(static_cast<size_t>(B) * Hv * 8);
  w.parts = reinterpret_cast<float*>(p);
  w.n_waves = n_waves;
  return w;
}

hipError_t launch_decode(const CacheView& c, const uint16_t* q, const int32_t* ctx,
                         const int32_t* slot, const int32_t* page_table, int pt_stride, int B,
                         int Hq, float scale_log2, float* out, float* lse,
                         const DecodeWorkspace& ws, const DecodeDebug* dbg, hipStream_t s,
                         hipEvent_t ev_main_begin, hipEvent_t ev_main_end, bool mx,
                         const uint16_t* k_new,
                         const uint16_t* v_new, const int32_t* pos_new) {
  // the fused append needs protected workgroups that own the new token
  if (k_new && (mx || c.window <= 0)) return hipErrorInvalidValue;
  if (ws.n_waves <= 0 || ws.n_waves % 4 != 0) return hipErrorInvalidValue;
  if (mx && dbg) return hipErrorInvalidValue;  // no debug instantiation of the MXFP4 variant
  DecArgs a{};
  a.pages = c.pages;
  a.side_codes = c.side_codes;
  a.side_scales = c.side_scales;
  a.Hkv = c.Hkv;
  a.Hq = Hq;
  a.G = Hq / c.Hkv;
  a.R = (a.G + GQA - 1) / GQA;
  a.Hv = c.Hkv * a.R;
  a.B = B;
  a.q = reinterpret_cast<const uint32_t*>(q);
  a.ctx = ctx;
  a.slot = slot;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.k_new = reinterpret_cast<const uint32_t*>(k_new);
  a.v_new = reinterpret_cast<const uint32_t*>(v_new);
  a.pos_new = pos_new;
  a.sink = c.sink;
  a.window = c.window;
  a.scale_log2 = scale_log2;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  if (dbg) a.dbg = *dbg;
  // main-region workgroups, then one protected-region workgroup per (b, g)
  const int prot_groups = c.sink + c.window > 0 ? B * a.Hv : 0;
  const dim3 block(256), groups(a.Hv * B), grid(ws.n_waves / 4 + prot_groups);
  if (B > 256) hipLaunchKernelGGL(plan_kernel, dim3(1), block, 0, s, a);
  if (dbg) {
    hipLaunchKernelGGL((main_kernel<Kv4Format, true>), grid, block, 0, s, a);
    hipLaunchKernelGGL(merge_kernel, groups, block, 0, s, a);
  } else {
    if (ev_main_begin) {
      const hipError_t e = hipEventRecord(ev_main_begin, s);
      if (e != hipSuccess) return e;
    }
    if (mx) hipLaunchKernelGGL((main_kernel<MxFormat, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((main_kernel<Kv4Format, false>), grid, block, 0, s, a);
    if (ev_main_end) {
      const hipError_t e = hipEventRecord(ev_main_end, s);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(merge_kernel, groups, block, 0, s, a);
  }
  return hipGetLastError();
}

size_t chunk_workspace_bytes(int T, int Hq, int Hkv, int n_waves) {
  (void)Hq;
  (void)Hkv;
  (void)n_waves;
  // block bases [nseq + 1] (nseq <= T)
  return (static_cast<size_t>(T + 1) * 4 + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_chunk_attention(const CacheView& c, const uint16_t* q, const int32_t* cu,
                                  const int32_t* start, int nseq, int T, const int32_t* slot,
                                  const int32_t* page_table, int pt_stride, int Hq, float scale_log2,
                                  float* out, float* lse, void* ws_base, int n_waves,
                                  const DecodeDebug* dbg, hipStream_t s) {
  (void)n_waves;
  if (nseq > T) return hipErrorInvalidValue;
  return launch_prefill_blocked(c, q, cu, start, nseq, T, slot, page_table, pt_stride, Hq, scale_log2, out,
                                lse, static_cast<int32_t*>(ws_base), dbg, s);
}

hipError_t launch_kv8_decode(const uint8_t* pages, int Hkv, const uint16_t* q, const int32_t* ctx,
                             const int32_t* page_table, int pt_stride, int B, int Hq,
                             float scale_log2, float* out, float* lse, const DecodeWorkspace& ws,
                             const DecodeDebug* dbg, hipStream_t s) {
  if (ws.n_waves <= 0 || ws.n_waves % 4 != 0) return hipErrorInvalidValue;
  DecArgs a{};
  a.pages = pages;
  a.Hkv = Hkv;
  a.Hq = Hq;
  a.G = Hq / Hkv;
  a.R = (a.G + GQA - 1) / GQA;
  a.Hv = Hkv * a.R;
  a.B = B;
  a.q = reinterpret_cast<const uint32_t*>(q);
  a.ctx = ctx;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.sink = 0;  // every page in the streamed region, no protected partial
  a.window = 0;
  a.scale_log2 = scale_log2;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  if (dbg) a.dbg = *dbg;
  const dim3 block(256), groups(a.Hv * B), grid(ws.n_waves / 4);
  if (B > 256) hipLaunchKernelGGL(plan_kernel, dim3(1), block, 0, s, a);
  if (dbg) hipLaunchKernelGGL((main_kernel<Kv8Format, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((main_kernel<Kv8Format, false>), grid, block, 0, s, a);
  hipLaunchKernelGGL(merge_kernel, groups, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kv4
