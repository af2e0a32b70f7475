// Re-prefill attention, query-blocked (paper.rainbus.top summary, "方法步骤详情"
// step 1: carried prefixes are re-prefilled after a weight update; step 4:
// the hybrid attention).  Token p of a chunk attends [0, p] under the
// protected set of the cache as it stands (cache end E = the chunk's end):
// the sinks below p + 1 and the window positions [max(s, E - w), p] from the
// INT8 side rows, and the main region [s, min(p + 1, E - w)) from the INT4
// pages, every 16-position tile of it processed by the decode step's per-tile
// rule (integer QK, Delta/m after the dot, tile softmax with exp2s, P-operand
// codes with the V step folded in, integer PV, FP32 running merge).
//
// One workgroup per (block of 8 consecutive tokens of a chunk, query-head group
// of up to 4 heads of one kv-head), its 4 waves splitting the block's side-row
// groups and main tiles, each tile and side row read once for 8 tokens x 4
// heads.  Every product takes the 32 rows
// n = 4 * token + head as its N dimension and is computed transposed:
//   QK:  D^T[32 positions][32 rows] = K[positions][16 channels] q^T   (i8)
//   PV:  O^T[32 channels][32 rows]  = V^T[channels][16 positions] P^T (the
//        integer codes on the f16 MFMA, exact, for the main tiles; BF16 hi /
//        lo parts of the FP32 weights for the protected rows)
// so that lane (n, kg) (n = lane % 32, kg = lane / 32) owns row n: it holds
// D of slots 8 kg .. 8 kg + 7 of both tiles of a pair (the K rows are loaded
// in that order), reduces a tile's max over its own 8 values and its partner
// lane's, and its 8 P codes of a tile are already the B operand of the PV
// product.
// Both regions accumulate into one running state per row (an exact
// log-sum-exp merge); the 4 waves' states merge through LDS into out, lse.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace kv4 {
namespace {

constexpr int QB = 8;             // query tokens per block
constexpr int NR = QB * GQA;      // 32 rows
constexpr int kQRowBytes = HD;    // query codes of a row in LDS: even channels, then odd
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) uint8_t* gbytes;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// The main tiles' PV product comes out of the f16 MFMA as the integer sum
// times 2^-20.
constexpr float kPvScale = 1048576.0f;

// How far (base 2) a pair's max may pass a row's reference max before the
// reference moves and the running state is rescaled.
constexpr float kLazyZ = 8.0f;

// Slot of a tile (0..15) that row m' of its half of the QK product holds:
// register r of lane (n, kg) holds rows 8 (r / 4) + 4 kg + r % 4, i.e. slots
// 8 kg + 4 ((r / 4) % 2) + r % 4 of tile r / 8, so that the lane's 8 values of
// a tile are slots 8 kg .. 8 kg + 7 in order.
__device__ __forceinline__ int tile_slot(int m) { return 8 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Two floats holding integers below 2048 as an f16 pair (exact).
__device__ __forceinline__ h2 f16_pair(float a, float b) {
  return __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(a, b));
}

struct PaArgs {
  const uint8_t* pages;
  const int8_t* side_codes;
  const uint16_t* side_scales;
  int Hkv, Hq, sink, window;
  int G, R, Hv;       // query heads per kv-head, groups of up to 4 per kv-head, groups per token
  const uint32_t* q;  // BF16 pairs [T][Hq][64]
  const int32_t* cu;
  const int32_t* start;
  const int32_t* slot;  // [nseq] side-buffer slot of each sequence (null: the sequence index)
  const int32_t* page_table;
  int pt_stride, nseq;
  const int32_t* blk_base;  // [nseq + 1] first block of each sequence
  float scale_log2;
  float* out;
  float* lse;
  DecodeDebug dbg;
};

template <typename T>
__device__ __forceinline__ T ldc(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Block base of each sequence: blk_base[s] = sum over earlier sequences of
// ceil(n / 8) (one workgroup).
__global__ __launch_bounds__(256) void block_base_kernel(const int32_t* __restrict__ cu, int nseq,
                                                         int32_t* blk_base) {
  __shared__ int32_t scan[256];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nseq; base += 256) {
    const int s = base + threadIdx.x;
    scan[threadIdx.x] = s < nseq ? (cu[s + 1] - cu[s] + QB - 1) / QB : 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int t = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += t;
      __syncthreads();
    }
    if (s < nseq) blk_base[s + 1] = carry + scan[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 255) carry += scan[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) blk_base[0] = 0;
}

__device__ __forceinline__ long lo_nib64(long x) { return x & 0x0F0F0F0F0F0F0F0FL; }
__device__ __forceinline__ long hi_nib64(long x) {
  return static_cast<long>((static_cast<unsigned long>(x) >> 4) & 0x0F0F0F0F0F0F0F0FUL);
}

// The swap of lanes l and l + 32 leaves, in every lane, its own value in one
// result and its partner's in the other.
__device__ __forceinline__ float partner_max(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Max of the 8 values of one tile held by this lane (registers 8 t' .. 8 t' + 7)
// and those of the partner lane (same row, other kg).
__device__ __forceinline__ float tile_max8(const float* v) {
  float m = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
  return partner_max(m);
}
// Smallest of 8 values, NaN if any is NaN (v_minimum3_f32).
__device__ __forceinline__ float z_lo8(const float* v) {
  float m = __builtin_elementwise_minimum(__builtin_elementwise_minimum(v[0], v[1]), v[2]);
  m = __builtin_elementwise_minimum(__builtin_elementwise_minimum(m, v[3]), v[4]);
  m = __builtin_elementwise_minimum(__builtin_elementwise_minimum(m, v[5]), v[6]);
  return __builtin_elementwise_minimum(m, v[7]);
}
__device__ __forceinline__ float partner_sum(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

constexpr int kLdsQ = 0;                                // [32 rows][128] query codes (even | odd)
constexpr int kLdsQi = kLdsQ + NR * kQRowBytes;         // [32] c_q, [32] S_q
constexpr int kPartRow = HD + 4;                        // padded row of a partial in LDS (floats)
constexpr int kLdsPart = kLdsQi + 2 * NR * 4;           // [4 waves][32 rows][kPartRow] A
constexpr int kLdsZL = kLdsPart + 4 * NR * kPartRow * 4;  // [4 waves][32 rows] Z, then l
constexpr int kLdsBytes = kLdsZL + 2 * 4 * NR * 4;

template <bool DEBUG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(PaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  // query-head group v: kv-head g, query heads h0 .. h0 + nh - 1 (rows of a
  // head past nh repeat head h0 + nh - 1 and are never stored)
  const int v = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.Hv));
  const int g = v / a.R;
  const int h0 = g * a.G + GQA * (v - g * a.R), nh = min(GQA, a.G - (h0 - g * a.G));
  const int total = ldc(a.blk_base + a.nseq);
  const int rev = static_cast<int>(blockIdx.x / static_cast<unsigned>(a.Hv));
  if (rev >= total) return;
  const int bq = total - 1 - rev;  // later (longer) blocks first
  int lo = 0, hi = a.nseq;         // blk_base[lo] <= bq < blk_base[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ldc(a.blk_base + mid) <= bq) lo = mid;
    else hi = mid;
  }
  const int sq = lo;
  const int lb = bq - ldc(a.blk_base + sq);
  const int cu0 = ldc(a.cu + sq), n_s = ldc(a.cu + sq + 1) - cu0;
  const int st0 = ldc(a.start + sq);
  const int tok0 = cu0 + QB * lb;
  const int ntok = min(QB, n_s - QB * lb);
  const int p0 = st0 + QB * lb;  // position of the block's first token
  const int E = st0 + n_s;       // cache end

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, kg = lane >> 5;  // row n = 4 * token + head
  int8_t* qlds = reinterpret_cast<int8_t*>(lds + kLdsQ);
  float* cq_l = reinterpret_cast<float*>(lds + kLdsQi);
  float* sq_l = cq_l + NR;

  // ---- queries: rotate, symmetric INT8 (rows 8 wave .. 8 wave + 7; lane l
  // holds channels 2l, 2l+1), codes to LDS as even channels then odd
#pragma unroll 1
  for (int k = 0; k < QB; ++k) {
    const int row = QB * wave + k;
    const int ti = row >> 2, h = row & 3;
    int c0 = 0, c1 = 0;
    float s_q = 0.0f;
    if (ti < ntok) {
      const size_t bh = static_cast<size_t>(tok0 + ti) * a.Hq + h0 + min(h, nh - 1);
      const uint32_t qw = a.q[bh * 64 + lane];
      float x0 = bf16_lo(qw), x1 = bf16_hi(qw);
      fwht128_wave(x0, x1);
      const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      s_q = amax / 127.0f;
      if (s_q != 0.0f) {
        c0 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x0 / s_q), -127.0f), 127.0f));
        c1 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x1 / s_q), -127.0f), 127.0f));
      }
      if (DEBUG && a.dbg.qcodes && h < nh) {
        a.dbg.qcodes[bh * HD + 2 * lane] = static_cast<int8_t>(c0);
        a.dbg.qcodes[bh * HD + 2 * lane + 1] = static_cast<int8_t>(c1);
      }
    }
    const int S = wave_sum_i(c0 + c1);
    if (DEBUG && a.dbg.qsum && lane == 0 && ti < ntok && h < nh)
      a.dbg.qsum[static_cast<size_t>(tok0 + ti) * a.Hq + h0 + h] = S;
    qlds[row * kQRowBytes + lane] = static_cast<int8_t>(c0);
    qlds[row * kQRowBytes + 64 + lane] = static_cast<int8_t>(c1);
    if (lane == 0) {
      cq_l[row] = s_q * a.scale_log2;
      sq_l[row] = static_cast<float>(S);
    }
  }
  __syncthreads();
  // B operands of QK: MFMA (c, parity) takes channels 32 c + 16 kg + 2 i + parity
  long qb[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      qb[c][par] = *reinterpret_cast<const long*>(qlds + n * kQRowBytes + 64 * par + 16 * c + 8 * kg);
  const float c_q = cq_l[n], S_q = sq_l[n];
  const int tn = n >> 2;  // token of this lane's row
  const bool row_live = tn < ntok;
  const int me_row = row_live ? min(p0 + tn + 1, E - a.window) : 0;  // main region end of the row

  // ---- main tiles of the block: [s / 16, (me_max - 1) / 16], in pairs
  const int me_max = min(p0 + ntok, E - a.window);
  const int j_lo = a.sink / PAGE;
  const int n_tiles = me_max > a.sink ? (me_max - 1) / PAGE - j_lo + 1 : 0;
  const int n_pairs = (n_tiles + 1) >> 1;
  const int pr0 = n_pairs * wave / 4, pr1 = n_pairs * (wave + 1) / 4;
  const int32_t* ptrow = a.page_table + static_cast<size_t>(sq) * a.pt_stride;
  const size_t pstride = static_cast<size_t>(a.Hkv) * BLOCK_BYTES;
  const gbytes gbase = (gbytes)a.pages + static_cast<size_t>(g) * BLOCK_BYTES;

  v16f O[4];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) O[s2] = v16f{};
  float Zr = -INFINITY, Ls = 0.0f, Ms = 0.0f;

  // ---- protected region: side rows [0, n_side) in groups of 32 (group k on
  // wave k % 4), INT8 QK^T on the same query operands (side K bytes split into
  // even and odd channels), FP32 weights, v^ = bf16(s_v c) and PV^T on the
  // BF16 MFMA with each weight as the sum of two BF16 parts (hi = bf16(e),
  // lo = bf16(e - hi): 16 significant bits), accumulated into the same
  // running state as the main tiles (an exact log-sum-exp merge of the two
  // regions)
  const int p_last = p0 + ntok - 1;
  const bool any_window = a.window > 0 && p_last >= max(a.sink, E - a.window);
  const int n_side = any_window ? a.sink + a.window : min(a.sink, p_last + 1);
  const int slot = a.slot ? ldc(a.slot + sq) : sq;
  const size_t srow0 = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS;
#pragma unroll 1
  for (int kgp = wave; 32 * kgp < n_side; kgp += 4) {
    const int r0 = 32 * kgp;
    // A operands of QK^T: side row r0 + n (loads clamped to the buffer)
    const gbytes krow = (gbytes)a.side_codes + (srow0 + min(r0 + n, SIDE_ROWS - 1)) * 2 * HD;
    long sa[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u4v x = *reinterpret_cast<const __attribute__((address_space(1))) u4v*>(krow + 32 * c + 16 * kg);
      const uint32_t e0 = __builtin_amdgcn_perm(x[1], x[0], 0x06040200u), e1 = __builtin_amdgcn_perm(x[3], x[2], 0x06040200u);
      const uint32_t o0 = __builtin_amdgcn_perm(x[1], x[0], 0x07050301u), o1 = __builtin_amdgcn_perm(x[3], x[2], 0x07050301u);
      sa[c][0] = static_cast<long>(e0) | (static_cast<long>(e1) << 32);
      sa[c][1] = static_cast<long>(o0) | (static_cast<long>(o1) << 32);
    }
    // (s_k, s_v) of the lane's side rows r0 + 8 j4 + 4 kg .. + 3
    u4v sc[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
      sc[j4] = *reinterpret_cast<const __attribute__((address_space(1))) u4v*>(
          (gbytes)a.side_scales + (srow0 + min(r0 + 8 * j4 + 4 * kg, SIDE_ROWS - 4)) * 4);
    v16i d = {};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d = __builtin_amdgcn_mfma_i32_32x32x16_i8(sa[c][0], qb[c][0], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_i32_32x32x16_i8(sa[c][1], qb[c][1], d, 0, 0, 0);
    }
    float z[16];
    float zm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rs = r0 + 8 * (r >> 2) + 4 * kg + (r & 3);
      const int pos = row_live ? side_position(rs, p0 + tn + 1, E, a.sink, a.window) : -1;
      const float sk = f16_value(sc[r >> 2][r & 3] & 0xFFFFu);
      z[r] = pos >= 0 ? (static_cast<float>(d[r]) * sk) * c_q : -INFINITY;
      zm = fmaxf(zm, z[r]);
      if (DEBUG && pos >= 0 && a.dbg.qk && (n & 3) < nh) {
        const size_t bh = static_cast<size_t>(tok0 + tn) * a.Hq + h0 + (n & 3);
        a.dbg.qk[bh * a.dbg.max_ctx + pos] = d[r];
      }
    }
    const float Zn = fmaxf(Zr, partner_max(zm));
    const float al = Zr == Zn ? 1.0f : __builtin_amdgcn_exp2f(Zr - Zn);
    Zr = Zn;
    if (__builtin_amdgcn_ballot_w64(al != 1.0f)) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) O[s2] *= al;
    }
    Ls *= al;
    Ms *= al;
    // weights as BF16 hi / lo parts, B operands of PV^T per chunk j4
    v4s ehi[4], elo[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float hv[4], lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2s(z[4 * j4 + i] - Zn);
        Ls += e;
        hv[i] = round_bf16(e);
        lv[i] = e - hv[i];
      }
      ehi[j4] = v4s{static_cast<short>(__float_as_uint(hv[0]) >> 16), static_cast<short>(__float_as_uint(hv[1]) >> 16),
                    static_cast<short>(__float_as_uint(hv[2]) >> 16), static_cast<short>(__float_as_uint(hv[3]) >> 16)};
      elo[j4] = v4s{static_cast<short>(__float_as_uint(round_bf16(lv[0])) >> 16),
                    static_cast<short>(__float_as_uint(round_bf16(lv[1])) >> 16),
                    static_cast<short>(__float_as_uint(round_bf16(lv[2])) >> 16),
                    static_cast<short>(__float_as_uint(round_bf16(lv[3])) >> 16)};
    }
    // A operands of PV^T: v^ of channel 32 s2 + n for side rows r0 + 8 j4 +
    // 4 kg .. + 3; rows no token of the block sees are zero (their bytes may
    // be stale)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float sv[4];
      int rr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rs = r0 + 8 * j4 + 4 * kg + i;
        const bool seen = side_position(rs, p_last + 1, E, a.sink, a.window) >= 0;
        sv[i] = seen ? f16_value(sc[j4][i] >> 16) : 0.0f;
        rr[i] = min(rs, SIDE_ROWS - 1);
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int8_t cv = *reinterpret_cast<const __attribute__((address_space(1))) int8_t*>(
              (gbytes)a.side_codes + ((srow0 + rr[i]) * 2 + 1) * HD + 32 * s2 + n);
          x[i] = round_bf16(sv[i] * static_cast<float>(cv));  // s_v c is exact in FP32
        }
        const v4s va = v4s{static_cast<short>(__float_as_uint(x[0]) >> 16), static_cast<short>(__float_as_uint(x[1]) >> 16),
                           static_cast<short>(__float_as_uint(x[2]) >> 16), static_cast<short>(__float_as_uint(x[3]) >> 16)};
        O[s2] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(va, ehi[j4], O[s2], 0, 0, 0);
        O[s2] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(va, elo[j4], O[s2], 0, 0, 0);
      }
    }
  }

  // A pair every row sees whole (all 8 tokens live, both tiles below the
  // first token's main end) skips the masks.
  const int me_min = min(p0 + 1, E - a.window);
  // The loads of a pair: K codes (A operands of QK: row m of the pair is tile
  // m / 16, slot tile_slot(m % 16), code bytes 16 c + 8 kg .. + 7), V codes (A
  // operands of PV per tile t and channel block s2: channel 32 s2 + n, the 4
  // code bytes of slots 8 kg .. 8 kg + 7) and the (delta, m) of the lane's
  // positions (registers 4 j4 .. 4 j4 + 3 hold rows 8 j4 + 4 kg .. + 3 of the
  // pair, i.e. tile j4 / 2, slots 8 kg + 4 (j4 % 2) .. + 3).
  struct PairData {
    long ka[4];
    uint32_t vw[2][4];
    u4v kmeta[4], vmeta[4];
  };
  auto pair_load = [&](int pr) {
    PairData L;
    const int ja = j_lo + 2 * pr;
    const bool has_b = 2 * pr + 1 < n_tiles;
    const int pta = ldc(ptrow + ja);
    const int ptb = has_b ? ldc(ptrow + ja + 1) : pta;
    const gbytes blk[2] = {gbase + static_cast<size_t>(static_cast<uint32_t>(pta)) * pstride,
                           gbase + static_cast<size_t>(static_cast<uint32_t>(ptb)) * pstride};
    const gbytes kb = blk[n >> 4] + 64 * tile_slot(n & 15);
#pragma unroll
    for (int c = 0; c < 4; ++c) L.ka[c] = *reinterpret_cast<const __attribute__((address_space(1))) long*>(kb + 16 * c + 8 * kg);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        L.vw[t][s2] = *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(
            blk[t] + OFF_VCODE + 8 * (32 * s2 + n) + 4 * kg);
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const gbytes mb = blk[j4 >> 1] + 4 * (8 * kg + 4 * (j4 & 1));
      L.kmeta[j4] = *reinterpret_cast<const __attribute__((address_space(1))) u4v*>(mb + OFF_KMETA);
      L.vmeta[j4] = *reinterpret_cast<const __attribute__((address_space(1))) u4v*>(mb + OFF_VMETA);
    }
    return L;
  };
  auto pair_step = [&](int pr, const PairData& L, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int ja = j_lo + 2 * pr;
    const bool has_b = 2 * pr + 1 < n_tiles;
    const long* ka = L.ka;
    const auto& vw = L.vw;
    const u4v* kmeta = L.kmeta;
    const u4v* vmeta = L.vmeta;
    // integer QK^T of the pair
    v16i d = {};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d = __builtin_amdgcn_mfma_i32_32x32x16_i8(lo_nib64(ka[c]), qb[c][0], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_i32_32x32x16_i8(hi_nib64(ka[c]), qb[c][1], d, 0, 0, 0);
    }
    float z[16], e[16], u[16];
    float emv_t[2], e_t[2];
    bool valid[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j4 = r >> 2, i = r & 3;
      const int t = j4 >> 1;
      const int slot16 = 8 * kg + 4 * (j4 & 1) + i;
      const int pos = PAGE * (ja + t) + slot16;
      valid[r] = FULL || (row_live && (t == 0 || has_b) && pos < me_row);
      const uint32_t km = kmeta[j4][i];
      const float dk = f16_value(km & 0xFFFFu);
      z[r] = valid[r] ? __builtin_fmaf(dk, static_cast<float>(d[r]), mul_f16(S_q, km >> 16)) * c_q : -INFINITY;
      if (DEBUG && valid[r] && a.dbg.qk && (n & 3) < nh) {
        const size_t bh = static_cast<size_t>(tok0 + tn) * a.Hq + h0 + (n & 3);
        a.dbg.qk[bh * a.dbg.max_ctx + pos] = d[r];
      }
    }
    const float zmax[2] = {tile_max8(&z[0]), tile_max8(&z[8])};
    // weights, u = e Delta_v, the tile sums l and sum(e m_v), and u_max
    float umax[2];
    auto tile_weights = [&](auto normal_tag) {
      constexpr bool NORMAL = decltype(normal_tag)::value;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float um = 0.0f;
        e_t[t] = -0.0f;  // -0 + e = e: no add for the first term
        emv_t[t] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 8 * t + k;
          const int j4 = r >> 2, i = r & 3;
          e[r] = NORMAL ? exp2s_normal(z[r] - zmax[t]) : exp2s(z[r] - zmax[t]);
          const uint32_t vm = vmeta[j4][i];
          // (metadata of positions outside the region may be any bits: selected away)
          u[r] = valid[r] ? mul_f16(e[r], vm & 0xFFFFu) : 0.0f;
          e_t[t] += valid[r] ? e[r] : 0.0f;
          emv_t[t] = valid[r] ? __builtin_fmaf(e[r], f16_value(vm >> 16), emv_t[t]) : emv_t[t];
          um = fmaxf(um, u[r]);
        }
        umax[t] = partner_max(um);
      }
    };
    if constexpr (FULL) {
      // exp2s selects 0 below -125.  When no logit of the pair lies more than
      // 125 below its tile's max (each lane tests the smallest of its 8 of
      // each tile; a NaN fails the test) the select is left out.
      const bool narrow = z_lo8(&z[0]) - zmax[0] >= -125.0f && z_lo8(&z[8]) - zmax[1] >= -125.0f;
      if (!__builtin_amdgcn_ballot_w64(!narrow)) tile_weights(std::true_type{});
      else tile_weights(std::false_type{});
    } else {
      tile_weights(std::false_type{});
    }
    // P codes; B operand of PV per tile, slot k of the lane's register k
    // (slot 8 kg + k of the tile), in the V operand's order: halves
    // (k, k + 4) for k = 0..3, the even k scaled by 16 (they meet the V codes
    // read at 1/16 of the odd slots' scale)
    h8 pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float qx = 127.0f / umax[t];
      const float inv = umax[t] == 0.0f ? 0.0f : qx;
      float pc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pc[k] = __builtin_amdgcn_fmed3f(__builtin_rintf(u[8 * t + k] * inv), 0.0f, 127.0f);
        if (DEBUG && valid[8 * t + k] && a.dbg.pcode && (n & 3) < nh) {
          const int pos = PAGE * (ja + t) + 8 * kg + k;
          const size_t bh = static_cast<size_t>(tok0 + tn) * a.Hq + h0 + (n & 3);
          a.dbg.pcode[bh * a.dbg.max_ctx + pos] = static_cast<uint8_t>(pc[k]);
        }
      }
      const h2 sixteen = {16.0f16, 16.0f16};
      const h2 p0 = f16_pair(pc[0], pc[4]) * sixteen, p1 = f16_pair(pc[1], pc[5]);
      const h2 p2 = f16_pair(pc[2], pc[6]) * sixteen, p3 = f16_pair(pc[3], pc[7]);
      pb[t] = h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
    // Running reference Z of the row: it moves to the pair's max only when
    // that passes it by more than kLazyZ, so the tile weights exp2(z_max - Z)
    // stay below 2^kLazyZ and what is accumulated is rescaled rarely (the
    // log-sum-exp merge is exact for any reference).  A row with no valid
    // position yet keeps Z = -inf and moves at its first finite max.
    const float Zm = fmaxf(zmax[0], zmax[1]);
    const bool move = Zm > Zr + kLazyZ;
    const float al = move ? __builtin_amdgcn_exp2f(Zr - Zm) : 1.0f;
    Zr = move ? Zm : Zr;
    if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) O[s2] *= al;
    }
    Ls *= al;
    Ms *= al;
    float wsu[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float wt = zmax[t] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(zmax[t] - Zr);
      Ls = __builtin_fmaf(wt, e_t[t], Ls);
      Ms = __builtin_fmaf(wt, emv_t[t], Ms);
      wsu[t] = wt * (umax[t] * (kPvScale / 127.0f));  // (u_max / 127) * 2^20: exact rescale
    }
    // integer PV^T per tile and channel block, on the f16 MFMA: V codes enter
    // as f16 subnormals (bits c -> c 2^-24, or 16 c 2^-24 for a high nibble
    // left in place), P codes as f16 integers; every product and partial sum
    // is an integer multiple of 2^-24 below 2^24 ulps, so the FP32 result is
    // the integer sum times 2^-20, exactly
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        // byte b of x holds slots 8 kg + 2 b (low nibble) and 8 kg + 2 b + 1
        const uint32_t x = vw[t][s2], y = x >> 8;
        const h8 va = __builtin_bit_cast(h8, u4v{x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u});
        const v16f acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[t], v16f{}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) O[s2][r] = __builtin_fmaf(wsu[t], acc[r], O[s2][r]);
        if (DEBUG && a.dbg.pv && row_live && (t == 0 || has_b) && (n & 3) < nh) {
          const size_t bh = static_cast<size_t>(tok0 + tn) * a.Hq + h0 + (n & 3);
          // a tile outside this row's main region leaves its accumulators unwritten
          if (PAGE * (ja + t) < me_row) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ch = 32 * s2 + 8 * (r >> 2) + 4 * kg + (r & 3);
              a.dbg.pv[(bh * a.dbg.max_pages + (ja + t)) * HD + ch] = static_cast<int32_t>(acc[r] * kPvScale);
            }
          }
        }
      }
    }
    };
  // The pairs every row sees whole (all 8 tokens live, 2 pr + 2 <= n_tiles
  // and PAGE (j_lo + 2 pr + 2) <= me_min) are a prefix of the wave's pairs;
  // one loop each keeps the running state in the same registers throughout.
  const int lim = min(n_tiles, me_min >= 0 ? me_min / PAGE - j_lo : -1);
  const int pf = ntok == QB && lim >= 2 ? max(pr0, min(pr1, lim >> 1)) : pr0;
  // Whole pairs: the next pair's loads go out before this pair's arithmetic
  // (two register sets in turn; past the end the last pair is loaded again).
  if (pr0 < pf) {
    PairData A = pair_load(pr0);
#pragma unroll 1
    for (int pr = pr0;; pr += 2) {
      const PairData B = pair_load(min(pr + 1, pf - 1));
      pair_step(pr, A, std::true_type{});
      if (pr + 1 >= pf) break;
      A = pair_load(min(pr + 2, pf - 1));
      pair_step(pr + 1, B, std::true_type{});
      if (pr + 2 >= pf) break;
    }
  }
#pragma unroll 1
  for (int pr = pf; pr < pr1; ++pr) pair_step(pr, pair_load(pr), std::false_type{});

  // ---- this wave's partial: A = O + sum(w e m_v), Z, l (rows n; both lanes
  // of a row hold half of the sums)
  const float Lrow = partner_sum(Ls), Mrow = partner_sum(Ms);
  float* part = reinterpret_cast<float*>(lds + kLdsPart) + (wave * NR + n) * kPartRow;
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[32 * s2 + 8 * (r >> 2) + 4 * kg + (r & 3)] = O[s2][r] + Mrow;
  float* zl = reinterpret_cast<float*>(lds + kLdsZL);
  if (kg == 0) {
    zl[wave * NR + n] = Zr;
    zl[4 * NR + wave * NR + n] = Lrow;
  }
  __syncthreads();

  // ---- exact merge of the 4 main partials and the protected partial of each
  // row (wave w: rows 8 w .. 8 w + 7; lane l: channels 2l, 2l+1)
  const float* partr = reinterpret_cast<const float*>(lds + kLdsPart);
#pragma unroll 1
  for (int k = 0; k < QB; ++k) {
    const int row = QB * wave + k;
    const int ti = row >> 2, h = row & 3;
    if (ti >= ntok || h >= nh) continue;
    const size_t bh = static_cast<size_t>(tok0 + ti) * a.Hq + h0 + h;
    float Zs[4], Lv[4];
    float2 Av[4];
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      Zs[w2] = zl[w2 * NR + row];
      Lv[w2] = zl[4 * NR + w2 * NR + row];
      Av[w2] = *reinterpret_cast<const float2*>(partr + (w2 * NR + row) * kPartRow + 2 * lane);
    }
    float Z = Zs[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) Z = fmaxf(Z, Zs[i]);
    float l = 0.0f;
    float2 A = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w = Zs[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Zs[i] - Z);
      l = __builtin_fmaf(w, Lv[i], l);
      A.x = __builtin_fmaf(w, Av[i].x, A.x);
      A.y = __builtin_fmaf(w, Av[i].y, A.y);
    }
    reinterpret_cast<float2*>(a.out + bh * HD)[lane] = make_float2(A.x / l, A.y / l);
    if (lane == 0) a.lse[bh] = 0.69314718055994531f * (Z + __builtin_log2f(l));
  }
}

}  // namespace

hipError_t launch_prefill_blocked(const CacheView& c, const uint16_t* q, const int32_t* cu,
                                  const int32_t* start, int nseq, int T, const int32_t* slot,
                                  const int32_t* page_table, int pt_stride, int Hq, float scale_log2,
                                  float* out, float* lse, int32_t* blk_base, const DecodeDebug* dbg,
                                  hipStream_t s) {
  if (nseq <= 0 || T <= 0) return hipErrorInvalidValue;
  PaArgs a{};
  a.pages = c.pages;
  a.side_codes = c.side_codes;
  a.side_scales = c.side_scales;
  a.Hkv = c.Hkv;
  a.Hq = Hq;
  a.G = Hq / c.Hkv;
  a.R = (a.G + GQA - 1) / GQA;
  a.Hv = c.Hkv * a.R;
  a.sink = c.sink;
  a.window = c.window;
  a.q = reinterpret_cast<const uint32_t*>(q);
  a.cu = cu;
  a.start = start;
  a.slot = slot;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.nseq = nseq;
  a.blk_base = blk_base;
  a.scale_log2 = scale_log2;
  a.out = out;
  a.lse = lse;
  if (dbg) a.dbg = *dbg;
  hipLaunchKernelGGL(block_base_kernel, dim3(1), dim3(256), 0, s, cu, nseq, blk_base);
  // blocks: sum of ceil(n / 8) <= (T + 7 nseq) / 8
  const long long nblk = (static_cast<long long>(T) + 7LL * nseq) / QB;
  const long long groups = nblk * a.Hv;
  if (groups > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(groups)), block(256);
  if (dbg) hipLaunchKernelGGL((prefill_attn_kernel<true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((prefill_attn_kernel<false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kv4
