// kv4_device.hpp -- device-side building blocks shared by the KV4-RL kernels
// (gfx950, wave64).  Numeric rules follow the KV4-RL pages (paper.rainbus.top
// summary, "分组仿射 KV 量化" and "方法步骤详情" steps 2-4); where the pages are
// silent the rule is stated where it is implemented.
#pragma once

#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kv4 {

constexpr int HD = 128;          // one quantization group = one 128-dim token-head vector
constexpr int PAGE = 16;         // positions per page
constexpr int SIDE_ROWS = 144;   // side-buffer rows per (slot, kv-head): sink + window <= 144
constexpr int BLOCK_BYTES = 2176;  // per (page, kv-head): 16 x (64 + 64 + 4 + 4)
constexpr int OFF_VCODE = 1024;
constexpr int OFF_KMETA = 2048;
constexpr int OFF_VMETA = 2112;
constexpr int GQA = 4;           // query heads per group (the rows of the kernels' operands)
// KV8-everywhere pool block per (page, kv-head): K codes [16][128] | V codes
// [128][16] | s_k FP16 [16] | s_v FP16 [16]
constexpr int KV8_BLOCK_BYTES = 4160;
constexpr int KV8_OFF_V = 2048;
constexpr int KV8_OFF_SK = 4096;
constexpr int KV8_OFF_SV = 4128;

// Position held by side row r of a cache ending at E, for sinks [0, s) and a
// ring of w recent positions in rows [s, s+w), if a query attending [0, L)
// sees it (-1 otherwise).
__device__ __forceinline__ int side_position(int r, int L, int E, int s, int w) {
  if (r < s) return r < L ? r : -1;
  if (r >= s + w) return -1;
  const int base = max(s, E - w);
  const int p = base + ((r - s - base) % w + w) % w;
  return p < L ? p : -1;
}

// ---------------------------------------------------------------- formats --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// IEEE binary16, round to nearest even (v_cvt_f16_f32 under the default mode,
// subnormals kept).
__device__ __forceinline__ uint32_t f16_bits(float x) {
  _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_value(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// x times the FP16 value with bits h, rounded once (the FP32 product of x and
// the exactly widened h), as an FMA with a +0 addend so that the compiler
// folds the widening into one v_fma_mix_f32 (with -0 it would become a plain
// multiply after a separate conversion).  The addend only turns a -0 product
// into +0; every caller's result is the same for either zero.
__device__ __forceinline__ float mul_f16(float x, uint32_t h) { return __builtin_fmaf(x, f16_value(h), 0.0f); }

// Round a finite binary32 to bfloat16 (nearest, ties to even); value kept in FP32.
__device__ __forceinline__ float round_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(u);
}

// ----------------------------------------------------------- cross-lane --

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// All-reduce over each row of 16 lanes: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror.  Every lane ends with the result.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp_f32<0xB1>(v));
  v = fminf(v, dpp_f32<0x4E>(v));
  v = fminf(v, dpp_f32<0x141>(v));
  v = fminf(v, dpp_f32<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

// Same all-reduce for non-negative floats, on their bit patterns (which order
// like unsigned integers), so each step is one fused DPP v_max_u32.
// row16_max for finite or -inf values on order-preserving integer keys (the
// bits for x >= +0, the bits with the low 31 flipped below, compared as
// signed), so that each stage is one DPP max; the same result except that a
// zero maximum is always +0.
__device__ __forceinline__ float row16_max_ord(float v) {
  int k = __float_as_int(v);
  k ^= (k >> 31) & 0x7FFFFFFF;
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0xB1, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x4E, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x141, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x140, 0xF, 0xF, true));
  k ^= (k >> 31) & 0x7FFFFFFF;
  return __int_as_float(k);
}
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, true)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, true)));
  return v;
}

// Value of lane 4*(l/4) + I in every lane l (quad_perm [I,I,I,I]).
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), I * 0x55, 0xF, 0xF, true));
}

// Read memory that no wave writes during the kernel (inputs, or outputs of an
// earlier launch) through the constant address space: wave-uniform reads then
// become scalar loads, which do not wait behind the vector loads in flight.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Value of lane l ^ H in every lane l (H = 1, 2, 4, 8, 16, 32) without LDS
// traffic: DPP quad permutations for 1 and 2, the swizzle crossbar for 4, a
// DPP rotation of the 16-lane row by 8 for 8, and the row-pair and half swaps
// (which leave every lane's own value in one result and its partner's in the
// other) for 16 and 32.
template <int H>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  static_assert(H == 1 || H == 2 || H == 4 || H == 8 || H == 16 || H == 32, "lane distance");
  if constexpr (H == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));
  } else if constexpr (H == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));
  } else if constexpr (H == 4) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x101F));  // xor 4 in 32 lanes
  } else if constexpr (H == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, true));
  } else if constexpr (H == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? s[0] : s[1];
  } else {
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? s[0] : s[1];
  }
}
template <int H>
__device__ __forceinline__ float xor_lane_f(float v) {
  return __uint_as_float(xor_lane<H>(__float_as_uint(v)));
}
template <int H>
__device__ __forceinline__ int xor_lane_i(int v) {
  return static_cast<int>(xor_lane<H>(static_cast<uint32_t>(v)));
}

// Wave-wide all-reductions, partners at lane distances 32, 16, ..., 1.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane_f<32>(v));
  v = fmaxf(v, xor_lane_f<16>(v));
  v = fmaxf(v, xor_lane_f<8>(v));
  v = fmaxf(v, xor_lane_f<4>(v));
  v = fmaxf(v, xor_lane_f<2>(v));
  return fmaxf(v, xor_lane_f<1>(v));
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, xor_lane_f<32>(v));
  v = fminf(v, xor_lane_f<16>(v));
  v = fminf(v, xor_lane_f<8>(v));
  v = fminf(v, xor_lane_f<4>(v));
  v = fminf(v, xor_lane_f<2>(v));
  return fminf(v, xor_lane_f<1>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane_f<32>(v);
  v += xor_lane_f<16>(v);
  v += xor_lane_f<8>(v);
  v += xor_lane_f<4>(v);
  v += xor_lane_f<2>(v);
  return v + xor_lane_f<1>(v);
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// row of 16 lanes (DPP row_shr, zero shifted in), then the totals of the
// rows below added from lanes 15, 31 and 47.  No LDS round trips.
__device__ __forceinline__ int wave_incl_sum_i(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += xor_lane_i<32>(v);
  v += xor_lane_i<16>(v);
  v += xor_lane_i<8>(v);
  v += xor_lane_i<4>(v);
  v += xor_lane_i<2>(v);
  return v + xor_lane_i<1>(v);
}

// ------------------------------------------------------------- rotation --
// Orthonormal Sylvester Hadamard H_128/sqrt(128) applied to a row vector held
// by one wave, lane l holding elements 2l (x0) and 2l+1 (x1).  FP32 in-place
// fast Walsh-Hadamard transform with element strides 1, 2, ..., 64 in that
// order, butterfly (a, b) -> (a + b, a - b), then one multiply by fp32(2^-3.5).
// The stride order fixes the FP32 sum tree of every output.
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;

// One butterfly stage across lanes: the lower lane of a pair keeps x + p, the
// upper one p - x, both written as p + (+-x) with the sign flipped by an xor
// (exact), so that the partner's value can enter the add as a DPP operand.
template <int H>
__device__ __forceinline__ void fwht_lane_stage(float& x0, float& x1) {
  const uint32_t flip = (threadIdx.x & H) ? 0x80000000u : 0u;
  x0 = xor_lane_f<H>(x0) + __uint_as_float(__float_as_uint(x0) ^ flip);
  x1 = xor_lane_f<H>(x1) + __uint_as_float(__float_as_uint(x1) ^ flip);
}
__device__ __forceinline__ void fwht128_wave(float& x0, float& x1) {
  const float a = x0 + x1, b = x0 - x1;
  x0 = a;
  x1 = b;
  fwht_lane_stage<1>(x0, x1);  // element stride 2h lives h lanes away
  fwht_lane_stage<2>(x0, x1);
  fwht_lane_stage<4>(x0, x1);
  fwht_lane_stage<8>(x0, x1);
  fwht_lane_stage<16>(x0, x1);
  fwht_lane_stage<32>(x0, x1);
  x0 = x0 * kInvSqrt128;
  x1 = x1 * kInvSqrt128;
}

// The same rotation with a row of 16 lanes per vector: lane r16 of the row
// holds elements 8 r16 .. 8 r16 + 7 in x[0..7]; strides 1, 2, 4 inside the
// lane, then 8, 16, 32, 64 across lanes (lane distances 1, 2, 4, 8), in that
// order, then the 2^-3.5 scale (the same sum tree as fwht128_wave).
__device__ __forceinline__ void fwht128_row16(float x[8], int r16) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const float u = x[j], v = x[j + h];
        x[j] = u + v;
        x[j + h] = u - v;
      }
  auto stage = [&](auto m_tag) {  // p + (+-x), as in fwht_lane_stage
    constexpr int M = decltype(m_tag)::value;
    const uint32_t flip = (r16 & M) ? 0x80000000u : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = xor_lane_f<M>(x[j]) + __uint_as_float(__float_as_uint(x[j]) ^ flip);
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = x[j] * kInvSqrt128;
}

// ----------------------------------------------------------- quantizers --

// Quotient RN(a/d) for a binary32 dividend and a divisor d with at most 11
// significant bits (an FP16 value), given y = RN(1/d).  a/d is then never
// closer than 2^-12 ulp to a rounding midpoint of binary32 (and never on
// one), the residual a - d*RN(a*y) is exact in one FMA, and q0 + r*y is within
// 2^-22 ulp of a/d, so a single rounding of it is the correctly rounded
// quotient.  This holds when a and a/d are normal; in the subnormal corner
// the last bits may differ, but such quotients are far below 1/2, so the
// integer codes taken from them do not.  Three operations instead of a full
// IEEE division sequence.
__device__ __forceinline__ float div_short_divisor(float a, float d, float y) {
  const float q0 = a * y;
  const float r = __builtin_fmaf(-q0, d, a);
  return __builtin_fmaf(r, y, q0);
}

// Group-affine INT4 metadata of one vector from its FP32 min and max:
// delta = fp16((max - min) / 15), offset m = fp16(min).
struct Int4Meta {
  uint32_t d16, m16;  // FP16 bit patterns
  float d, m;         // their values
  float dinv;         // RN(1/d), 0 when d == 0
};
__device__ __forceinline__ Int4Meta int4_meta(float mn, float mx) {
  Int4Meta r;
  const float range = mx - mn;
  r.d16 = f16_bits(range / 15.0f);
  r.m16 = f16_bits(mn);
  r.d = f16_value(r.d16);
  r.m = f16_value(r.m16);
  r.dinv = (r.d == 0.0f) ? 0.0f : 1.0f / r.d;
  return r;
}
// c = clamp(rint((x - m) / delta), 0, 15); a zero delta gives code 0.
__device__ __forceinline__ uint32_t int4_code(float x, const Int4Meta& q) {
  const float t = __builtin_rintf(div_short_divisor(x - q.m, q.d, q.dinv));
  const uint32_t c = static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), 15.0f));
  return q.d == 0.0f ? 0u : c;  // a select, not a branch per element
}

// Symmetric INT8 side copy: s = fp16(max|x| / 127), c = clamp(rint(x / s), -127, 127).
struct Int8Meta {
  uint32_t s16;
  float s, sinv;
};
__device__ __forceinline__ Int8Meta int8_meta(float amax) {
  Int8Meta r;
  r.s16 = f16_bits(amax / 127.0f);
  r.s = f16_value(r.s16);
  r.sinv = (r.s == 0.0f) ? 0.0f : 1.0f / r.s;
  return r;
}
__device__ __forceinline__ int32_t int8_code(float x, const Int8Meta& q) {
  const float t = __builtin_rintf(div_short_divisor(x, q.s, q.sinv));
  const int32_t c = static_cast<int32_t>(fminf(fmaxf(t, -127.0f), 127.0f));
  return q.s == 0.0f ? 0 : c;
}

// ------------------------------------------------------ cache entries --
// One token of one kv-head, held by one wave (lane l: channels 2l, 2l+1; K
// already rotated).

// INT4 entry in slot t of its page block: K token-major (channel 2l in the low
// nibble of byte l), V channel-major (this position's nibble of bytes 8c + t/2
// for channels 2l, 2l+1; the neighbouring position's nibble is kept), and the
// FP16 (delta, m) pairs.  The K half and the V half are independent (two
// waves may write them); the two V bytes this lane rewrites are read first
// (v_bytes_of), which a caller may issue early, next to its other loads.
struct VBytes {
  uint8_t b0, b1;
};
__device__ __forceinline__ VBytes v_bytes_of(const uint8_t* blk, int t, int lane) {
  const uint8_t* vb0 = blk + OFF_VCODE + 8 * (2 * lane) + (t >> 1);
  return VBytes{vb0[0], vb0[8]};
}
__device__ __forceinline__ void write_int4_k(uint8_t* blk, int t, float k0, float k1, int lane) {
  const Int4Meta kq = int4_meta(wave_min(fminf(k0, k1)), wave_max(fmaxf(k0, k1)));
  blk[64 * t + lane] = static_cast<uint8_t>(int4_code(k0, kq) | (int4_code(k1, kq) << 4));
  if (lane == 0) *reinterpret_cast<uint32_t*>(blk + OFF_KMETA + 4 * t) = kq.d16 | (kq.m16 << 16);
}
__device__ __forceinline__ void write_int4_v(uint8_t* blk, int t, float v0, float v1, int lane, VBytes old) {
  const Int4Meta vq = int4_meta(wave_min(fminf(v0, v1)), wave_max(fmaxf(v0, v1)));
  const int sh = (t & 1) * 4;
  const uint32_t keep = (t & 1) ? 0x0Fu : 0xF0u;
  uint8_t* vb0 = blk + OFF_VCODE + 8 * (2 * lane) + (t >> 1);
  vb0[0] = static_cast<uint8_t>((old.b0 & keep) | (int4_code(v0, vq) << sh));
  vb0[8] = static_cast<uint8_t>((old.b1 & keep) | (int4_code(v1, vq) << sh));
  if (lane == 0) *reinterpret_cast<uint32_t*>(blk + OFF_VMETA + 4 * t) = vq.d16 | (vq.m16 << 16);
}
__device__ __forceinline__ void write_int4_entry(uint8_t* blk, int t, float k0, float k1, float v0,
                                                 float v1, int lane) {
  write_int4_k(blk, t, k0, k1, lane);
  write_int4_v(blk, t, v0, v1, lane, v_bytes_of(blk, t, lane));
}

// INT8 side row: codes [2][128] (K then V), scales [2] FP16.  Returns this
// lane's two K and two V codes (byte pairs) and the scale bit patterns.
struct Int8Row {
  uint32_t kp, vp, ks16, vs16;
};
__device__ __forceinline__ Int8Row make_int8_row(float k0, float k1, float v0, float v1) {
  const Int8Meta ks = int8_meta(wave_max(fmaxf(fabsf(k0), fabsf(k1))));
  const Int8Meta vs = int8_meta(wave_max(fmaxf(fabsf(v0), fabsf(v1))));
  Int8Row r;
  r.kp = (static_cast<uint32_t>(int8_code(k0, ks)) & 0xFFu) | ((static_cast<uint32_t>(int8_code(k1, ks)) & 0xFFu) << 8);
  r.vp = (static_cast<uint32_t>(int8_code(v0, vs)) & 0xFFu) | ((static_cast<uint32_t>(int8_code(v1, vs)) & 0xFFu) << 8);
  r.ks16 = ks.s16;
  r.vs16 = vs.s16;
  return r;
}
__device__ __forceinline__ void store_int8_row(int8_t* codes, uint16_t* scales, const Int8Row& r, int lane) {
  reinterpret_cast<uint16_t*>(codes)[lane] = static_cast<uint16_t>(r.kp);
  reinterpret_cast<uint16_t*>(codes)[64 + lane] = static_cast<uint16_t>(r.vp);
  if (lane == 0) {
    scales[0] = static_cast<uint16_t>(r.ks16);
    scales[1] = static_cast<uint16_t>(r.vs16);
  }
}
__device__ __forceinline__ Int8Row write_int8_row(int8_t* codes, uint16_t* scales, float k0, float k1,
                                                  float v0, float v1, int lane) {
  const Int8Row r = make_int8_row(k0, k1, v0, v1);
  store_int8_row(codes, scales, r, lane);
  return r;
}

// ----------------------------------------------------------------- exp2 --
// Softmax weights: 2^y for y <= 0 evaluated the same way on every device so
// that P-operand codes are reproducible: y < -125 gives 0; otherwise
// n = rint(y), f = y - n (exact), degree-7 Taylor polynomial of 2^f in Horner
// form with FMA, coefficients RN(ln2^k / k!), result p * 2^n.
namespace detail {
constexpr double kLn2 = 0.6931471805599453094172321214581766;
constexpr float kC0 = 1.0f;
constexpr float kC1 = static_cast<float>(kLn2);
constexpr float kC2 = static_cast<float>(kLn2 * kLn2 / 2.0);
constexpr float kC3 = static_cast<float>(kLn2 * kLn2 * kLn2 / 6.0);
constexpr float kC4 = static_cast<float>(kLn2 * kLn2 * kLn2 * kLn2 / 24.0);
constexpr float kC5 = static_cast<float>(kLn2 * kLn2 * kLn2 * kLn2 * kLn2 / 120.0);
constexpr float kC6 = static_cast<float>(kLn2 * kLn2 * kLn2 * kLn2 * kLn2 * kLn2 / 720.0);
constexpr float kC7 = static_cast<float>(kLn2 * kLn2 * kLn2 * kLn2 * kLn2 * kLn2 * kLn2 / 5040.0);
}  // namespace detail

// The steps of exp2s without its final select: equal to exp2s(y) for
// y >= -125.
__device__ __forceinline__ float exp2s_normal(float y) {
  using namespace detail;
  const float n = __builtin_rintf(y);
  const float f = y - n;
  float p = kC7;
  p = __builtin_fmaf(p, f, kC6);
  p = __builtin_fmaf(p, f, kC5);
  p = __builtin_fmaf(p, f, kC4);
  p = __builtin_fmaf(p, f, kC3);
  p = __builtin_fmaf(p, f, kC2);
  p = __builtin_fmaf(p, f, kC1);
  p = __builtin_fmaf(p, f, kC0);
  return __builtin_ldexpf(p, static_cast<int>(n));
}

__device__ __forceinline__ float exp2s(float y) {
  // below -125 (and for -inf) the polynomial runs on whatever y gives and
  // the select returns 0
  const bool live = (y >= -125.0f);
  const float r = exp2s_normal(y);
  return live ? r : 0.0f;
}

}  // namespace kv4
