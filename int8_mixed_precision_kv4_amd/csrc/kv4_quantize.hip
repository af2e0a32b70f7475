// kv4_quantize.hip -- quantize-on-append and bulk re-prefill of the KV4-RL
// cache (paper.rainbus.top summary, "方法步骤详情" steps 1-3).
//
// Each K vector is rotated (Hadamard after RoPE), then K and V are quantized
// independently to group-affine INT4 (one group per 128-dim token-head
// vector, FP16 delta and offset computed on line) into their page slot; the s
// sink positions and the w recent positions (s = 16, w = 128 by default) also
// get a symmetric INT8 copy in the side buffer, sinks in rows [0, s) and
// position p >= s in ring row s + (p mod w).  A position leaving the recent
// window keeps its INT4 entry; its ring row is simply reused.
#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace kv4 {
namespace {

struct QuantArgs {
  uint8_t* pages;
  int8_t* side_codes;
  uint16_t* side_scales;
  int Hkv;
  const uint32_t* k;  // bf16 pairs: lane l of a vector reads elements 2l, 2l+1
  const uint32_t* v;
  const int32_t* slot;
  const int32_t* page_table;
  int pt_stride;
  int sink, window;
};

// Side row of position p; only called for p < sink or window > 0.
__device__ __forceinline__ int side_row(const QuantArgs& a, int p) {
  return p < a.sink ? p : a.sink + (p % a.window);
}

// INT8 side row of one position (K rotated, V), held by one wave.
__device__ __forceinline__ void write_side_row(const QuantArgs& a, int slot, int g, int pos,
                                               float k0, float k1, float v0, float v1, int lane) {
  const size_t r = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS + side_row(a, pos);
  write_int8_row(a.side_codes + r * 2 * HD, a.side_scales + r * 2, k0, k1, v0, v1, lane);
}

// MXFP4 variant of the main-region entry (KV4-RL pages, comparison of 4-bit
// formats): OCP MX blocks of 32 channels (16 lanes), E = floor(log2 amax) - 2
// clamped to [-127, 127] (-127 for an all-zero block), codes = E2M1 of
// x / 2^E, nearest with ties to even and saturation at 6, by the hardware
// conversion at unit scale after an exact ldexp.  Block layout: K codes [16][64]
// | V codes [128][8] | K scales E8M0 [16][4] | V scales E8M0 [16][4].
constexpr int MX_OFF_KS = 2048, MX_OFF_VS = 2112;

struct MxCodes {
  uint32_t kbyte, v0, v1;  // K: channels 2l (low) and 2l+1; V: code of channel 2l, 2l+1
  uint32_t ke8, ve8;       // E8M0 bytes of this lane's block (channels 32(l/16) ..)
};
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return -127;
  const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);  // 0 for a subnormal: clamps
  return max(ef - 127 - 2, -127);
}
__device__ __forceinline__ uint32_t mx_pair(float x0, float x1, int E) {
  const float y0 = __builtin_ldexpf(x0, -E), y1 = __builtin_ldexpf(x1, -E);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu;
}
__device__ __forceinline__ MxCodes mx_codes(float k0, float k1, float v0, float v1) {
  const int ek = mx_exponent(row16_max(fmaxf(fabsf(k0), fabsf(k1))));
  const int ev = mx_exponent(row16_max(fmaxf(fabsf(v0), fabsf(v1))));
  MxCodes c;
  c.kbyte = mx_pair(k0, k1, ek);
  const uint32_t vb = mx_pair(v0, v1, ev);
  c.v0 = vb & 0xFu;
  c.v1 = vb >> 4;
  c.ke8 = static_cast<uint32_t>(ek + 127);
  c.ve8 = static_cast<uint32_t>(ev + 127);
  return c;
}

// One token per sequence; one wave per (kv-head, sequence).
template <bool MX>
__global__ __launch_bounds__(64) void append_kernel(QuantArgs a, const int32_t* __restrict__ pos_arr) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int pos = pos_arr[b];
  const int slot = a.slot ? a.slot[b] : b;
  const size_t vec = static_cast<size_t>(b) * a.Hkv + g;
  const uint32_t kw = a.k[vec * 64 + lane], vw = a.v[vec * 64 + lane];
  float k0 = bf16_lo(kw), k1 = bf16_hi(kw);
  const float v0 = bf16_lo(vw), v1 = bf16_hi(vw);
  fwht128_wave(k0, k1);  // keys are stored in the rotated basis

  const int phys = a.page_table[static_cast<size_t>(b) * a.pt_stride + (pos >> 4)];
  const int t = pos & (PAGE - 1);
  uint8_t* blk = a.pages + (static_cast<size_t>(phys) * a.Hkv + g) * BLOCK_BYTES;

  if constexpr (MX) {
    const MxCodes mc = mx_codes(k0, k1, v0, v1);
    const uint32_t kbyte = mc.kbyte, vc0 = mc.v0, vc1 = mc.v1;
    if ((lane & 15) == 0) {
      blk[MX_OFF_KS + 4 * t + (lane >> 4)] = static_cast<uint8_t>(mc.ke8);
      blk[MX_OFF_VS + 4 * t + (lane >> 4)] = static_cast<uint8_t>(mc.ve8);
    }
    // K: token-major, channel 2l in the low nibble of byte l
    blk[64 * t + lane] = static_cast<uint8_t>(kbyte);
    // V: channel-major, this position's nibble in bytes 8c + t/2 of channels 2l, 2l+1;
    // the other nibble belongs to the neighbouring position and is kept.
    const int sh = (t & 1) * 4;
    const uint32_t keep = (t & 1) ? 0x0Fu : 0xF0u;
    uint8_t* vb0 = blk + OFF_VCODE + 8 * (2 * lane) + (t >> 1);
    uint8_t* vb1 = vb0 + 8;
    *vb0 = static_cast<uint8_t>((*vb0 & keep) | (vc0 << sh));
    *vb1 = static_cast<uint8_t>((*vb1 & keep) | (vc1 << sh));
  } else {
    write_int4_entry(blk, t, k0, k1, v0, v1, lane);
  }
  if (pos < a.sink || a.window > 0) write_side_row(a, slot, g, pos, k0, k1, v0, v1, lane);
}

// Re-prefill: one workgroup owns one (page, kv-head) block of one sequence, so
// nibble bytes shared by neighbouring positions have a single writer.  Side
// rows are written only where appends would leave them in the final state:
// sinks, and the last w positions of the range (earlier ring rows would be
// overwritten within the same range anyway; none when w = 0).  A row of 16
// lanes quantizes one token (lane r16: channels 8 r16 .. 8 r16 + 7), so that
// one wave takes 4 tokens at once and the per-vector work (reductions,
// metadata) is shared by four times more data per instruction.  Same
// arithmetic as the append kernel: the same rotation sum tree, exact min /
// max, the same quantizer calls, hence the same bytes.
__device__ __forceinline__ void unpack_bf16x8(uint4 r, float x[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}
// Nibble codes of 8 channels: channel 8 r16 + j in bits 4j .. 4j+3 (byte i
// = channels 2i (low nibble) and 2i+1 of the lane's 8).
__device__ __forceinline__ uint32_t int4_codes8(const float x[8], const Int4Meta& q) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= int4_code(x[j], q) << (4 * j);
  return w;
}
__device__ __forceinline__ Int4Meta int4_meta_row16(const float x[8]) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, x[j]);
    mx = fmaxf(mx, x[j]);
  }
  return int4_meta(row16_min(mn), row16_max(mx));
}
__device__ __forceinline__ uint2 int8_codes8(const float x[8], const Int8Meta& q) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j >> 2] |= (static_cast<uint32_t>(int8_code(x[j], q)) & 0xFFu) << (8 * (j & 3));
  return make_uint2(w[0], w[1]);
}
__device__ __forceinline__ Int8Meta int8_meta_row16(const float x[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  return int8_meta(row16_max(amax));
}

// MXFP4 with 8 channels per lane: the block's max |x| over its 4 lanes (the
// quad of the DPP quad permutations), and the E2M1 codes of the lane's 8
// channels at unit scale after the exact ldexp by -E (low nibble first).
__device__ __forceinline__ float quad_max_abs8(const float x[8]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
  m = fmaxf(m, dpp_f32<0xB1>(m));
  return fmaxf(m, dpp_f32<0x4E>(m));
}
__device__ __forceinline__ uint32_t mx_codes8(const float x[8], int E) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= mx_pair(x[2 * i], x[2 * i + 1], E) << (8 * i);
  return w;
}

// 128 threads: row r (lanes 16r .. 16r+15) quantizes page slots r and r + 8,
// both tokens' K and V loaded before either is processed; MX selects the
// MXFP4 main-region entry instead of INT4.
template <bool MX>
__global__ __launch_bounds__(128) void prefill16_kernel(QuantArgs a, const int32_t* __restrict__ cu,
                                                        const int32_t* __restrict__ start_pos) {
  // the kv-heads of a page side by side in the grid
  const int g = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.Hkv));
  const int lp = static_cast<int>(blockIdx.x / static_cast<unsigned>(a.Hkv)), s = blockIdx.y;
  const int n = cu[s + 1] - cu[s];
  if (n <= 0) return;
  const int start = start_pos[s], end = start + n;
  const int page = (start >> 4) + lp;
  if (page > ((end - 1) >> 4)) return;
  const int t0 = max(start - page * PAGE, 0), t1 = min(end - page * PAGE, PAGE);
  const int slot = a.slot ? a.slot[s] : s;
  const int phys = a.page_table[static_cast<size_t>(s) * a.pt_stride + page];
  uint8_t* blk = a.pages + (static_cast<size_t>(phys) * a.Hkv + g) * BLOCK_BYTES;
  const int keep_from = max(a.sink, end - a.window);  // == end when w = 0

  __shared__ __attribute__((aligned(16))) uint8_t vcodes[PAGE][HD];
  const int r16 = threadIdx.x & 15;
  const int row = threadIdx.x >> 4;  // 0..7
  uint4 kr[2], vr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = row + 8 * u;
    kr[u] = vr[u] = make_uint4(0u, 0u, 0u, 0u);
    if (t >= t0 && t < t1) {
      const size_t vec = (static_cast<size_t>(cu[s]) + (page * PAGE + t - start)) * a.Hkv + g;
      kr[u] = reinterpret_cast<const uint4*>(a.k + vec * 64)[r16];
      vr[u] = reinterpret_cast<const uint4*>(a.v + vec * 64)[r16];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = row + 8 * u;  // page slot of this row
    const bool live = t >= t0 && t < t1;
    const int p = page * PAGE + t;
    float kx[8], vx[8];
    unpack_bf16x8(kr[u], kx);
    unpack_bf16x8(vr[u], vx);
    fwht128_row16(kx, r16);  // every row takes part in the cross-lane stages
    uint32_t kc, vc;  // nibble codes of the lane's 8 channels
    if constexpr (MX) {
      // MXFP4: 32-channel blocks = 4 lanes (block r16 / 4)
      const int ek = mx_exponent(quad_max_abs8(kx)), ev = mx_exponent(quad_max_abs8(vx));
      kc = mx_codes8(kx, ek);
      vc = mx_codes8(vx, ev);
      if (live && (r16 & 3) == 0) {
        blk[MX_OFF_KS + 4 * t + (r16 >> 2)] = static_cast<uint8_t>(ek + 127);
        blk[MX_OFF_VS + 4 * t + (r16 >> 2)] = static_cast<uint8_t>(ev + 127);
      }
    } else {
      const Int4Meta kq = int4_meta_row16(kx);
      const Int4Meta vq = int4_meta_row16(vx);
      kc = int4_codes8(kx, kq);
      vc = int4_codes8(vx, vq);
      if (live && r16 == 0) {
        *reinterpret_cast<uint32_t*>(blk + OFF_KMETA + 4 * t) = kq.d16 | (kq.m16 << 16);
        *reinterpret_cast<uint32_t*>(blk + OFF_VMETA + 4 * t) = vq.d16 | (vq.m16 << 16);
      }
    }
    if (live) {
      *reinterpret_cast<uint32_t*>(blk + 64 * t + 4 * r16) = kc;
      // V codes of the slot, one byte per channel, for the channel-major pass
      uint2 vb;
      vb.x = (vc & 0xFu) | (((vc >> 4) & 0xFu) << 8) | (((vc >> 8) & 0xFu) << 16) | (((vc >> 12) & 0xFu) << 24);
      vb.y = ((vc >> 16) & 0xFu) | (((vc >> 20) & 0xFu) << 8) | (((vc >> 24) & 0xFu) << 16) | ((vc >> 28) << 24);
      *reinterpret_cast<uint2*>(&vcodes[t][8 * r16]) = vb;
    }
    // INT8 side row: final sinks and the last w positions of the sequence
    const bool side = live && (p < a.sink || p >= keep_from);
    if (__builtin_amdgcn_ballot_w64(side)) {  // the row reductions need every lane of a row
      const Int8Meta ks = int8_meta_row16(kx), vs = int8_meta_row16(vx);
      if (side) {
        const size_t r = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS + side_row(a, p);
        int8_t* codes = a.side_codes + r * 2 * HD;
        *reinterpret_cast<uint2*>(codes + 8 * r16) = int8_codes8(kx, ks);
        *reinterpret_cast<uint2*>(codes + HD + 8 * r16) = int8_codes8(vx, vs);
        if (r16 == 0) {
          a.side_scales[r * 2] = static_cast<uint16_t>(ks.s16);
          a.side_scales[r * 2 + 1] = static_cast<uint16_t>(vs.s16);
        }
      }
    }
  }
  __syncthreads();
  // V codes, channel-major: per pass, thread -> channel j, positions 8*half ..
  // 8*half+7 (one dword); nibbles of positions outside [t0, t1) are kept.
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = threadIdx.x + 128 * pass;
    const int j = idx >> 1, half = idx & 1;
    uint32_t* vw = reinterpret_cast<uint32_t*>(blk + OFF_VCODE + 8 * j + 4 * half);
    const bool whole = (t0 <= 8 * half) && (t1 >= 8 * half + 8);
    uint32_t w = whole ? 0u : *vw;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tt = 8 * half + i;
      if (tt >= t0 && tt < t1) w = (w & ~(0xFu << (4 * i))) | (static_cast<uint32_t>(vcodes[tt][j]) << (4 * i));
    }
    *vw = w;
  }
}

// ---------------------------------------------- re-prefill, page per wave --
// One wave quantizes the 16 page slots of one (page, kv-head) block: lane
// (t = lane / 4, cg = lane % 4) holds token t's channels 32 i + 8 cg + k
// (chunk i = 0..3, k = 0..7) of K and of V, so the per-vector work (the
// min / max reductions, two of them across the lane quad, and the FP16
// metadata) is shared by 16 tokens per instruction, and the V codes of the
// whole page can be turned channel-major inside the wave.  Rotation: FWHT
// strides 1, 2, 4 over k, 8 and 16 across the quad (lane distances 1 and 2),
// 32 and 64 over i, in that order, then the 2^-3.5 scale: the sum tree of
// fwht128_wave.  Codes come from the same division and rounding as
// int4_code; a zero delta has a zero reciprocal, so the quotient is 0 and
// the codes are 0 with no select.  Side rows as in prefill16_kernel.

// FP32 in-lane butterflies over the chunk index bits (h = 8 for stride 32,
// 16 for stride 64) or over k (h = 1, 2, 4): element j pairs with j + h.
template <int H>
__device__ __forceinline__ void fwht_inlane(float x[32]) {
#pragma unroll
  for (int j = 0; j < 32; ++j)
    if ((j & H) == 0) {
      const float u = x[j], v = x[j + H];
      x[j] = u + v;
      x[j + H] = u - v;
    }
}
__device__ __forceinline__ void fwht128_quad(float x[32]) {
  fwht_inlane<1>(x);
  fwht_inlane<2>(x);
  fwht_inlane<4>(x);
#pragma unroll
  for (int j = 0; j < 32; ++j) {  // strides 8 and 16: partner lanes lane ^ 1, lane ^ 2
    const uint32_t flip = (threadIdx.x & 1) ? 0x80000000u : 0u;
    x[j] = xor_lane_f<1>(x[j]) + __uint_as_float(__float_as_uint(x[j]) ^ flip);
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t flip = (threadIdx.x & 2) ? 0x80000000u : 0u;
    x[j] = xor_lane_f<2>(x[j]) + __uint_as_float(__float_as_uint(x[j]) ^ flip);
  }
  fwht_inlane<8>(x);
  fwht_inlane<16>(x);
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = x[j] * kInvSqrt128;
}

// min / max over the 128 channels of the lane quad's token
__device__ __forceinline__ Int4Meta int4_meta_quad(const float x[32]) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 32; ++j) {
    mn = fminf(mn, x[j]);
    mx = fmaxf(mx, x[j]);
  }
  mn = fminf(mn, dpp_f32<0xB1>(mn));
  mn = fminf(mn, dpp_f32<0x4E>(mn));
  mx = fmaxf(mx, dpp_f32<0xB1>(mx));
  mx = fmaxf(mx, dpp_f32<0x4E>(mx));
  return int4_meta(mn, mx);
}
__device__ __forceinline__ Int8Meta int8_meta_quad(const float x[32]) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) a = fmaxf(a, fabsf(x[j]));
  a = fmaxf(a, dpp_f32<0xB1>(a));
  a = fmaxf(a, dpp_f32<0x4E>(a));
  return int8_meta(a);
}

// INT4 code of x as a float in {0, ..., 15}: rint((x - m) / delta) clamped.
__device__ __forceinline__ float int4_code_f(float x, const Int4Meta& q) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(div_short_divisor(x - q.m, q.d, q.dinv)), 0.0f, 15.0f);
}
// Chunk of 8 channels -> 8 nibbles (channel k of the chunk in bits 4k..4k+3):
// four codes at a time are combined as c0 + 16 c1 + 256 c2 + 4096 c3, exact
// in FP32, before one conversion.
__device__ __forceinline__ uint32_t int4_chunk(const float* x, const Int4Meta& q) {
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = int4_code_f(x[k], q);
  const float lo = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c[3], 16.0f, c[2]), 16.0f, c[1]), 16.0f, c[0]);
  const float hi = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c[7], 16.0f, c[6]), 16.0f, c[5]), 16.0f, c[4]);
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}
__device__ __forceinline__ uint2 int8_chunk(const float* x, const Int8Meta& q) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k >> 2] |= (static_cast<uint32_t>(int8_code(x[k], q)) & 0xFFu) << (8 * (k & 3));
  return make_uint2(w[0], w[1]);
}

// 256 threads = 4 waves, wave w takes kv-head 4 blockIdx.x % hq4 + w of page
// blockIdx.x / hq4 of sequence blockIdx.y (hq4 = ceil(Hkv / 4)).
__global__ __launch_bounds__(256) void prefill_page_kernel(QuantArgs a, const int32_t* __restrict__ cu,
                                                           const int32_t* __restrict__ start_pos) {
  const int hq4 = (a.Hkv + 3) >> 2;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int g = 4 * static_cast<int>(blockIdx.x % static_cast<unsigned>(hq4)) + wave;
  const int lp = static_cast<int>(blockIdx.x / static_cast<unsigned>(hq4)), s = blockIdx.y;
  if (g >= a.Hkv) return;  // wave-uniform; the kernel has no workgroup barrier
  const int n = cu[s + 1] - cu[s];
  if (n <= 0) return;
  const int start = start_pos[s], end = start + n;
  const int page = (start >> 4) + lp;
  if (page > ((end - 1) >> 4)) return;
  const int t0 = max(start - page * PAGE, 0), t1 = min(end - page * PAGE, PAGE);
  const int t = lane >> 2, cg = lane & 3;
  const bool live = t >= t0 && t < t1;
  const int slot = a.slot ? a.slot[s] : s;
  const int phys = a.page_table[static_cast<size_t>(s) * a.pt_stride + page];
  uint8_t* blk = a.pages + (static_cast<size_t>(phys) * a.Hkv + g) * BLOCK_BYTES;
  const int keep_from = max(a.sink, end - a.window);  // == end when w = 0

  // token t's K and V: 16-byte chunk 4 i + cg holds channels 32 i + 8 cg ..
  // (lanes of slots outside [t0, t1) point at slot t0 and load nothing)
  uint4 kr[4], vr[4];
  {
    const int tl = live ? t : t0;
    const size_t vec = (static_cast<size_t>(cu[s]) + (page * PAGE + tl - start)) * a.Hkv + g;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k + vec * 64);
    const uint4* vp = reinterpret_cast<const uint4*>(a.v + vec * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = live ? kp[4 * i + cg] : make_uint4(0u, 0u, 0u, 0u);
      vr[i] = live ? vp[4 * i + cg] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float kx[32], vx[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unpack_bf16x8(kr[i], kx + 8 * i);
    unpack_bf16x8(vr[i], vx + 8 * i);
  }
  fwht128_quad(kx);  // keys are stored in the rotated basis

  const Int4Meta kq = int4_meta_quad(kx);
  const Int4Meta vq = int4_meta_quad(vx);
  uint32_t kc[4], vc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kc[i] = int4_chunk(kx + 8 * i, kq);
    vc[i] = int4_chunk(vx + 8 * i, vq);
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(blk + 64 * t + 16 * i + 4 * cg) = kc[i];
    if (cg == 0) {
      *reinterpret_cast<uint32_t*>(blk + OFF_KMETA + 4 * t) = kq.d16 | (kq.m16 << 16);
      *reinterpret_cast<uint32_t*>(blk + OFF_VMETA + 4 * t) = vq.d16 | (vq.m16 << 16);
    }
  }
  // INT8 side row: final sinks and the last w positions of the sequence
  const int p = page * PAGE + t;
  const bool side = live && (p < a.sink || p >= keep_from);
  if (__builtin_amdgcn_ballot_w64(side)) {  // the quad reductions need every lane of a quad
    const Int8Meta ks = int8_meta_quad(kx), vs = int8_meta_quad(vx);
    if (side) {
      const size_t r = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS + side_row(a, p);
      int8_t* codes = a.side_codes + r * 2 * HD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint2*>(codes + 32 * i + 8 * cg) = int8_chunk(kx + 8 * i, ks);
        *reinterpret_cast<uint2*>(codes + HD + 32 * i + 8 * cg) = int8_chunk(vx + 8 * i, vs);
      }
      if (cg == 0) {
        a.side_scales[r * 2] = static_cast<uint16_t>(ks.s16);
        a.side_scales[r * 2 + 1] = static_cast<uint16_t>(vs.s16);
      }
    }
  }

  // V codes channel-major through the wave's 1 KB of LDS: written token-major
  // (row t = 64 bytes, channel 2b in the low nibble of byte b), then lane L
  // gathers byte L of the 16 rows (channels 2L, 2L+1 of every slot) and
  // splits the nibbles into the two channels' 8-byte runs.
  __shared__ __attribute__((aligned(16))) uint8_t vt[4][PAGE * 64];
  uint8_t* tl = vt[wave];
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(tl + 64 * t + 16 * i + 4 * cg) = vc[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // bytes of slots 4m .. 4m+3, then the low nibbles of slot pairs (2k, 2k+1)
    // into bytes 0 and 2, and the high nibbles likewise
    const uint32_t d = static_cast<uint32_t>(tl[64 * (4 * m) + lane]) |
                       (static_cast<uint32_t>(tl[64 * (4 * m + 1) + lane]) << 8) |
                       (static_cast<uint32_t>(tl[64 * (4 * m + 2) + lane]) << 16) |
                       (static_cast<uint32_t>(tl[64 * (4 * m + 3) + lane]) << 24);
    const uint32_t x = d & 0x0F0F0F0Fu, z = d & 0xF0F0F0F0u;
    lo[m] = x | (x >> 4);
    hi[m] = (z >> 4) | (z >> 8);
  }
  // channel 2L: bytes 0 and 2 of lo[0..3]; channel 2L + 1: the same of hi
  uint4 out;
  out.x = __builtin_amdgcn_perm(lo[1], lo[0], 0x06040200u);
  out.y = __builtin_amdgcn_perm(lo[3], lo[2], 0x06040200u);
  out.z = __builtin_amdgcn_perm(hi[1], hi[0], 0x06040200u);
  out.w = __builtin_amdgcn_perm(hi[3], hi[2], 0x06040200u);
  uint4* dst = reinterpret_cast<uint4*>(blk + OFF_VCODE + 16 * lane);
  if (t0 > 0 || t1 < PAGE) {  // a partial page keeps the other slots' nibbles
    uint32_t keep0 = 0u, keep1 = 0u;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      keep0 |= (tt >= t0 && tt < t1) ? 0u : (0xFu << (4 * tt));
      keep1 |= (tt + 8 >= t0 && tt + 8 < t1) ? 0u : (0xFu << (4 * tt));
    }
    const uint4 old = *dst;
    out.x = (out.x & ~keep0) | (old.x & keep0);
    out.y = (out.y & ~keep1) | (old.y & keep1);
    out.z = (out.z & ~keep0) | (old.z & keep0);
    out.w = (out.w & ~keep1) | (old.w & keep1);
  }
  *dst = out;
}

// ------------------------------------------------------------ KV8 pool --
// KV8 everywhere (the INT8 comparison variant): every position in the side
// rows' representation (rotated key, symmetric INT8 per 128-dim vector, FP16
// scale), in a paged pool whose block per (page, kv-head) is K codes
// [16][128] token-major | V codes [128][16] channel-major | s_k[16] | s_v[16].
// Every byte belongs to one position, so tokens are written independently.

struct Kv8Args {
  uint8_t* pages;
  int Hkv;
  const uint32_t* k;
  const uint32_t* v;
  const int32_t* page_table;
  int pt_stride;
};

__device__ __forceinline__ void kv8_write(const Kv8Args& a, int g, int phys, int t, uint32_t kw,
                                          uint32_t vw, int lane) {
  float k0 = bf16_lo(kw), k1 = bf16_hi(kw);
  const float v0 = bf16_lo(vw), v1 = bf16_hi(vw);
  fwht128_wave(k0, k1);
  const Int8Meta ks = int8_meta(wave_max(fmaxf(fabsf(k0), fabsf(k1))));
  const Int8Meta vs = int8_meta(wave_max(fmaxf(fabsf(v0), fabsf(v1))));
  uint8_t* blk = a.pages + (static_cast<size_t>(phys) * a.Hkv + g) * KV8_BLOCK_BYTES;
  reinterpret_cast<uint16_t*>(blk + HD * t)[lane] =
      static_cast<uint16_t>((static_cast<uint32_t>(int8_code(k0, ks)) & 0xFFu) |
                            ((static_cast<uint32_t>(int8_code(k1, ks)) & 0xFFu) << 8));
  blk[KV8_OFF_V + PAGE * (2 * lane) + t] = static_cast<uint8_t>(int8_code(v0, vs));
  blk[KV8_OFF_V + PAGE * (2 * lane + 1) + t] = static_cast<uint8_t>(int8_code(v1, vs));
  if (lane == 0) {
    reinterpret_cast<uint16_t*>(blk + KV8_OFF_SK)[t] = static_cast<uint16_t>(ks.s16);
    reinterpret_cast<uint16_t*>(blk + KV8_OFF_SV)[t] = static_cast<uint16_t>(vs.s16);
  }
}

// One token per sequence; one wave per (kv-head, sequence).
__global__ __launch_bounds__(64) void kv8_append_kernel(Kv8Args a, const int32_t* __restrict__ pos_arr) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int pos = pos_arr[b];
  const size_t vec = static_cast<size_t>(b) * a.Hkv + g;
  const int phys = a.page_table[static_cast<size_t>(b) * a.pt_stride + (pos >> 4)];
  kv8_write(a, g, phys, pos & (PAGE - 1), a.k[vec * 64 + lane], a.v[vec * 64 + lane], lane);
}

// Re-prefill: one wave per (token, kv-head); workgroup (x, g, s) covers
// tokens 4x .. 4x+3 of sequence s.
__global__ __launch_bounds__(256) void kv8_prefill_kernel(Kv8Args a, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ start_pos) {
  const int g = blockIdx.y, s = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = 4 * blockIdx.x + wave;
  if (i >= cu[s + 1] - cu[s]) return;
  const int p = start_pos[s] + i;
  const size_t vec = (static_cast<size_t>(cu[s]) + i) * a.Hkv + g;
  const int phys = a.page_table[static_cast<size_t>(s) * a.pt_stride + (p >> 4)];
  kv8_write(a, g, phys, p & (PAGE - 1), a.k[vec * 64 + lane], a.v[vec * 64 + lane], lane);
}

}  // namespace

hipError_t launch_kv8_append(uint8_t* pages, int Hkv, const uint16_t* k, const uint16_t* v,
                             const int32_t* pos, const int32_t* page_table, int pt_stride, int B,
                             hipStream_t s) {
  Kv8Args a{pages, Hkv, reinterpret_cast<const uint32_t*>(k), reinterpret_cast<const uint32_t*>(v),
            page_table, pt_stride};
  hipLaunchKernelGGL(kv8_append_kernel, dim3(Hkv, B), dim3(64), 0, s, a, pos);
  return hipGetLastError();
}

hipError_t launch_kv8_prefill(uint8_t* pages, int Hkv, const uint16_t* k, const uint16_t* v,
                              const int32_t* cu, const int32_t* start, const int32_t* page_table,
                              int pt_stride, int nseq, int max_seqlen, hipStream_t s) {
  Kv8Args a{pages, Hkv, reinterpret_cast<const uint32_t*>(k), reinterpret_cast<const uint32_t*>(v),
            page_table, pt_stride};
  hipLaunchKernelGGL(kv8_prefill_kernel, dim3((max_seqlen + 3) / 4, Hkv, nseq), dim3(256), 0, s, a,
                     cu, start);
  return hipGetLastError();
}

hipError_t launch_append(const CacheView& c, const uint16_t* k, const uint16_t* v,
                         const int32_t* pos, const int32_t* slot, const int32_t* page_table,
                         int pt_stride, int B, hipStream_t s, bool mx) {
  QuantArgs a{c.pages, c.side_codes, c.side_scales, c.Hkv,
              reinterpret_cast<const uint32_t*>(k), reinterpret_cast<const uint32_t*>(v),
              slot, page_table, pt_stride, c.sink, c.window};
  if (mx) hipLaunchKernelGGL(append_kernel<true>, dim3(c.Hkv, B), dim3(64), 0, s, a, pos);
  else hipLaunchKernelGGL(append_kernel<false>, dim3(c.Hkv, B), dim3(64), 0, s, a, pos);
  return hipGetLastError();
}

hipError_t launch_prefill(const CacheView& c, const uint16_t* k, const uint16_t* v,
                          const int32_t* cu, const int32_t* start, const int32_t* slot,
                          const int32_t* page_table, int pt_stride, int nseq, int max_seqlen,
                          hipStream_t s, bool mx) {
  QuantArgs a{c.pages, c.side_codes, c.side_scales, c.Hkv,
              reinterpret_cast<const uint32_t*>(k), reinterpret_cast<const uint32_t*>(v),
              slot, page_table, pt_stride, c.sink, c.window};
  const int pages = (max_seqlen + PAGE - 1) / PAGE + 1;
  if (mx) hipLaunchKernelGGL(prefill16_kernel<true>, dim3(pages * c.Hkv, nseq), dim3(128), 0, s, a, cu, start);
  else hipLaunchKernelGGL(prefill_page_kernel, dim3(pages * ((c.Hkv + 3) / 4), nseq), dim3(256), 0, s, a, cu,
                          start);
  return hipGetLastError();
}

}  // namespace kv4
