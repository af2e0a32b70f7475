// kv4_decode.hip -- one decode step of KV4-RL hybrid attention
// (paper.rainbus.top summary, "方法步骤详情" step 4 and "核心方法"; onedev.kr
// summary, "전제와 한계").
//
// Three launches on the caller's stream:
//   1. query_kernel, one workgroup per (kv-head, sequence): rotates and
//      INT8-quantizes the 4 queries of the group once for both regions.
//      Workgroup (0,0) also writes the work plan (prefix sums of main pages).
//   2. main_kernel, a fixed grid of independent waves: the concatenated list
//      of main-region pages of all (sequence, kv-head) pairs is cut into equal
//      contiguous chunks, one per wave (split-K with exact load balance).  Per
//      page: integer QK on MFMA (INT8 query x unpacked INT4 keys), delta/m
//      applied after the dot, tile softmax, INT8 P operand with the V scale
//      folded in, integer PV on MFMA, FP32 running merge.  A wave writes one
//      partial per (sequence, kv-head) segment it touches.
//   3. protected_kernel, one workgroup per (kv-head, sequence): INT8 QK
//      against the side keys, FP32 softmax, PV over BF16-dequantized side
//      values, then the exact log-sum-exp merge of this protected partial with
//      the main partials of the group, written as out and lse.
#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace kv4 {
namespace {

struct DecArgs {
  const uint8_t* pages;
  const int8_t* side_codes;
  const uint16_t* side_scales;
  int Hkv, Hq, B;
  const uint32_t* q;  // bf16 pairs
  const int32_t* ctx;
  const int32_t* slot;
  const int32_t* page_table;
  int pt_stride;
  float scale_log2;
  float* out;
  float* lse;
  DecodeWorkspace ws;
  DecodeDebug dbg;
};

// Main region M = [16, L-128) covers logical pages 1 .. (L-129)/16.
__device__ __forceinline__ int main_pages(int L) { return L > SIDE_ROWS ? (L - 129) / PAGE : 0; }

// plan[b] = sum over earlier sequences of main_pages * Hkv (one workgroup).
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
    scan[threadIdx.x] = (b < a.B) ? main_pages(a.ctx[b]) * a.Hkv : 0;
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

// Query codes in the workspace, per (sequence, q-head): 128 B in MFMA operand
// order (even channels, then odd channels) and 128 B in natural order.
constexpr int kQStride = 2 * HD;

template <bool DEBUG>
__global__ __launch_bounds__(256) void query_kernel(DecArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  if (g == 0 && b == 0) build_plan(a);
  const int h = g * GQA + wave;
  const size_t bh = static_cast<size_t>(b) * a.Hq + h;
  // Rotate the query like the keys, then symmetric INT8 with an FP32 scale.
  const uint32_t qw = a.q[bh * 64 + lane];
  float x0 = bf16_lo(qw), x1 = bf16_hi(qw);
  fwht128_wave(x0, x1);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s_q = amax / 127.0f;
  int c0 = 0, c1 = 0;
  if (s_q != 0.0f) {
    c0 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x0 / s_q), -127.0f), 127.0f));
    c1 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x1 / s_q), -127.0f), 127.0f));
  }
  const int S = wave_sum_i(c0 + c1);
  int8_t* qs = a.ws.qcodes + bh * kQStride;
  qs[lane] = static_cast<int8_t>(c0);
  qs[64 + lane] = static_cast<int8_t>(c1);
  reinterpret_cast<uint16_t*>(qs + HD)[lane] = static_cast<uint16_t>((c0 & 0xFF) | ((c1 & 0xFF) << 8));
  if (lane == 0) {
    a.ws.qinfo[bh * 4 + 0] = s_q * a.scale_log2;  // c_q: s_q, the scale and log2(e)
    a.ws.qinfo[bh * 4 + 1] = __int_as_float(S);
    a.ws.qinfo[bh * 4 + 2] = s_q;
    a.ws.qinfo[bh * 4 + 3] = 0.0f;
    if (DEBUG && a.dbg.qsum) a.dbg.qsum[bh] = S;
  }
  if (DEBUG && a.dbg.qcodes) {
    a.dbg.qcodes[bh * HD + 2 * lane] = static_cast<int8_t>(c0);
    a.dbg.qcodes[bh * HD + 2 * lane + 1] = static_cast<int8_t>(c1);
  }
}

// QK MFMA output has head v of position l%16 in register v of lanes 0..15;
// move head h to row h (lanes 16h..16h+15).
__device__ __forceinline__ int qk_rows(v4i d) {
  const auto r01 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(d[0]),
                                                    static_cast<uint32_t>(d[1]), false, false);
  const auto r23 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(d[2]),
                                                    static_cast<uint32_t>(d[3]), false, false);
  const auto r = __builtin_amdgcn_permlane32_swap(r01[0], r23[0], false, false);
  return static_cast<int>(r[0]);
}

// ------------------------------------------------------------------ main --

__device__ __forceinline__ uint32_t lo_nibbles(uint32_t x) { return x & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t hi_nibbles(uint32_t x) { return (x >> 4) & 0x0F0F0F0Fu; }
__device__ __forceinline__ v4i nib_lo(uint4 x) {
  return v4i{static_cast<int>(lo_nibbles(x.x)), static_cast<int>(lo_nibbles(x.y)),
             static_cast<int>(lo_nibbles(x.z)), static_cast<int>(lo_nibbles(x.w))};
}
__device__ __forceinline__ v4i nib_hi(uint4 x) {
  return v4i{static_cast<int>(hi_nibbles(x.x)), static_cast<int>(hi_nibbles(x.y)),
             static_cast<int>(hi_nibbles(x.z)), static_cast<int>(hi_nibbles(x.w))};
}
// 16 positions of one channel (8 nibble bytes) -> 16 INT8 operand bytes; byte
// i of the result holds position 8(i/8) + 2(i%4) + (i/4)%2.
__device__ __forceinline__ v4i nib_positions(uint32_t lo8, uint32_t hi8) {
  return v4i{static_cast<int>(lo_nibbles(lo8)), static_cast<int>(hi_nibbles(lo8)),
             static_cast<int>(lo_nibbles(hi8)), static_cast<int>(hi_nibbles(hi8))};
}
// inverse of that byte order
__device__ __forceinline__ int pcode_slot(int t) { return 8 * (t >> 3) + 4 * (t & 1) + ((t & 7) >> 1); }


// Per-wave LDS staging slot of one quad (4 pages of one segment):
//   [0, 4096)     K codes, tile t at 1024 t + 16 lane
//   [4096, 8192)  V codes, channel block s2 at 4096 + 1024 s2 + 16 lane
//   [8192, 8704)  metadata, page t at 8192 + 128 t: 16 x {delta, m} K, then V
// followed by 256 B where the P operand is assembled.
constexpr int kSlotK = 0, kSlotV = 4096, kSlotMeta = 8192, kSlotP = 8704, kSlotBytes = 8960;

struct QuadRegs {
  uint4 kq[4], vq[4];
  uint32_t km[4], vm[4];
};

// Issue the direct-to-LDS loads of one quad.  Tile t reads physical page
// blk[t]; lane (r16, grp) fetches K bytes 64 r16 + 16 grp of every tile, and V
// bytes 1024 + 16(16 s2 + r16) of tile grp (the k-group of the PV MFMA).
__device__ __forceinline__ void quad_to_lds(uint8_t* slot, const gptr blk[4], int lane, int r16,
                                            int grp) {
  const int koff = 64 * r16 + 16 * grp;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    __builtin_amdgcn_global_load_lds(blk[t] + koff, (lptr)(slot + kSlotK + 1024 * t), 16, 0, 0);
  const gptr vb = grp == 0 ? blk[0] : grp == 1 ? blk[1] : grp == 2 ? blk[2] : blk[3];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2)
    __builtin_amdgcn_global_load_lds(vb + OFF_VCODE + 16 * (16 * s2 + r16),
                                     (lptr)(slot + kSlotV + 1024 * s2), 16, 0, 0);
  if (lane < 32) {  // 4 pages x 128 B of metadata
    const int t = lane >> 3;
    const gptr mb = t == 0 ? blk[0] : t == 1 ? blk[1] : t == 2 ? blk[2] : blk[3];
    __builtin_amdgcn_global_load_lds(mb + OFF_KMETA + 16 * (lane & 7), (lptr)(slot + kSlotMeta), 16, 0, 0);
  }
}

__device__ __forceinline__ void quad_from_lds(QuadRegs& q, const uint8_t* slot, int lane, int r16) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    q.kq[t] = *reinterpret_cast<const uint4*>(slot + kSlotK + 1024 * t + 16 * lane);
    q.vq[t] = *reinterpret_cast<const uint4*>(slot + kSlotV + 1024 * t + 16 * lane);
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
template <bool DEBUG>
__device__ __forceinline__ void compute_quad(const DecArgs& a, MainState& st, const QuadRegs& q,
                                             int np, v4i qa0, v4i qa1, float c_q, float S_q,
                                             int j0, int main_end, size_t qb, uint8_t* stage,
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
    const bool valid = (t < np) && (pos < main_end);
    const float dk = f16_value(q.km[t] & 0xFFFFu), mk = f16_value(q.km[t] >> 16);
    const float dv = f16_value(q.vm[t] & 0xFFFFu), mv = f16_value(q.vm[t] >> 16);
    // q.k^ = s_q (delta * sum(qc*c) + m * sum(qc)); c_q carries s_q, the scale and log2(e)
    const float z = valid ? __builtin_fmaf(dk, static_cast<float>(D), mk * S_q) * c_q : -INFINITY;
    zmax[t] = row16_max(z);
    e[t] = valid ? exp2s(z - zmax[t]) : 0.0f;
    u[t] = valid ? e[t] * dv : 0.0f;    // V scale folded into P
    emv[t] = valid ? e[t] * mv : 0.0f;  // V offset applied after the dot
    umax[t] = __uint_as_float(row16_max_u32(__float_as_uint(u[t])));
    if (DEBUG && valid && a.dbg.qk) a.dbg.qk[(qb + grp) * a.dbg.max_ctx + pos] = D;
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
    if (DEBUG && a.dbg.pcode) {
      const int pos = PAGE * (j0 + t) + r16;
      if (t < np && pos < main_end) a.dbg.pcode[(qb + grp) * a.dbg.max_ctx + pos] = static_cast<uint8_t>(uc);
    }
  }
  // running reference max of each head; rescale what is accumulated
  const float Zn = fmaxf(st.Zr, fmaxf(fmaxf(zmax[0], zmax[1]), fmaxf(zmax[2], zmax[3])));
  const float al = __builtin_amdgcn_exp2f(st.Zr - Zn);
#pragma unroll
  for (int o = 0; o < 8; ++o) st.O[o] *= al;
  st.Ls *= al;
  st.Ms *= al;
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
      // lane: head grp, channel 2(16 s2 + r16) + e2, tile v in register v
      const int o = 2 * s2 + e2;
      float x = st.O[o];
      x = __builtin_fmaf(wsu[0], static_cast<float>(acc[0]), x);
      x = __builtin_fmaf(wsu[1], static_cast<float>(acc[1]), x);
      x = __builtin_fmaf(wsu[2], static_cast<float>(acc[2]), x);
      x = __builtin_fmaf(wsu[3], static_cast<float>(acc[3]), x);
      st.O[o] = x;
      if (DEBUG && a.dbg.pv) {
        const int ch = 2 * (16 * s2 + r16) + e2;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < np) a.dbg.pv[((qb + grp) * a.dbg.max_pages + (j0 + t)) * HD + ch] = acc[t];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <bool DEBUG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KV4_MAIN_WAVES_PER_SIMD, KV4_MAIN_WAVES_PER_SIMD))) void main_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][kSlotBytes];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * 4 + wave;
  const int nw = a.ws.n_waves;
  const int32_t* plan = a.ws.plan;
  const int64_t T = ld_const(plan + a.B);
  const int64_t start = static_cast<int64_t>(w) * T / nw;
  const int64_t end = static_cast<int64_t>(w + 1) * T / nw;
  if (start >= end) return;
  int lo = 0, hi = a.B;  // plan[lo] <= start < plan[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_const(plan + mid) <= start) lo = mid;
    else hi = mid;
  }
  int b = lo;
  uint8_t* slot = lds[wave];
  uint8_t* stage = slot + kSlotP;
  const int pslot = pcode_slot(r16);
  const size_t pstride = static_cast<size_t>(a.Hkv) * BLOCK_BYTES;
  int64_t page = start;

  while (page < end) {
    while (ld_const(plan + b + 1) <= page) ++b;
    const int pb = ld_const(plan + b);
    const int mp = (ld_const(plan + b + 1) - pb) / a.Hkv;
    const int g = static_cast<int>((page - pb) / mp);
    const int64_t seg0 = pb + static_cast<int64_t>(g) * mp;
    const int64_t stop = min(end, seg0 + mp);
    const int main_end = ld_const(a.ctx + b) - WINDOW;
    const size_t qb = static_cast<size_t>(b) * a.Hq + g * GQA;
    const int32_t* ptrow = a.page_table + static_cast<size_t>(b) * a.pt_stride;
    const gptr gbase = (gptr)a.pages + static_cast<size_t>(g) * BLOCK_BYTES;
    auto quad_np = [&](int64_t p) { return static_cast<int>(min(static_cast<int64_t>(4), stop - p)); };
    auto quad_j0 = [&](int64_t p) { return 1 + static_cast<int>(p - seg0); };
    auto issue = [&](int64_t p) {
      const int j0 = quad_j0(p), np = quad_np(p);
      gptr blk[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        blk[t] = gbase + static_cast<size_t>(ld_const(ptrow + j0 + min(t, np - 1))) * pstride;
      quad_to_lds(slot, blk, lane, r16, grp);
    };
    issue(page);  // first quad of the segment in flight during the set-up below

    // A operand of QK: rows 0..3 = the group's heads, k = channels
    // (lane group grp covers channels 32grp..32grp+31, even / odd split).
    v4i qa0 = {0, 0, 0, 0}, qa1 = {0, 0, 0, 0};
    if (r16 < GQA) {
      const int8_t* qs = a.ws.qcodes + (qb + r16) * kQStride;
      qa0 = *reinterpret_cast<const v4i*>(qs + 16 * grp);
      qa1 = *reinterpret_cast<const v4i*>(qs + 64 + 16 * grp);
    }
    const float c_q = ld_const(a.ws.qinfo + (qb + grp) * 4 + 0);
    const float S_q = static_cast<float>(__float_as_int(ld_const(a.ws.qinfo + (qb + grp) * 4 + 1)));
    MainState st;
    st.Zr = -INFINITY;
    st.Ls = 0.0f;
    st.Ms = 0.0f;
#pragma unroll
    for (int o = 0; o < 8; ++o) st.O[o] = 0.0f;

    // Pipeline: quad i is read out of the slot, quad i+1 streams into it
    // while quad i is computed.
    for (int64_t p0 = page; p0 < stop; p0 += 4) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      QuadRegs q;
      quad_from_lds(q, slot, lane, r16);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      if (p0 + 4 < stop) issue(p0 + 4);
      compute_quad<DEBUG>(a, st, q, quad_np(p0), qa0, qa1, c_q, S_q, quad_j0(p0), main_end, qb,
                          stage, r16, grp, pslot);
    }
    // partial of this (sequence, kv-head) segment: A = O + sum(w e m_v)
    const float Lh = row16_sum(st.Ls), Mh = row16_sum(st.Ms);
    const size_t bg = static_cast<size_t>(b) * a.Hkv + g;
    float* P = a.ws.parts + ((static_cast<size_t>(w) + bg) * GQA + grp) * kPart;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      *reinterpret_cast<float2*>(P + 2 * (16 * s2 + r16)) = make_float2(st.O[2 * s2] + Mh, st.O[2 * s2 + 1] + Mh);
    if (r16 == 0) {
      P[128] = st.Zr;
      P[129] = Lh;
    }
    page = stop;
  }
}

// ------------------------------------------------------------ protected --

// Position held by side row r when the context is L (-1: row not in use).
__device__ __forceinline__ int side_position(int r, int L) {
  if (r < SINK) return r < L ? r : -1;
  const int base = max(SINK, L - WINDOW);
  const int p = base + ((r - SINK - base) % WINDOW + WINDOW) % WINDOW;
  return p < L ? p : -1;
}

// Waves of the main grid whose page chunk contains page p of the plan (chunk
// c covers [c T / nw, (c+1) T / nw); empty chunks own nothing).
__device__ __forceinline__ int chunk_of(int64_t p, int64_t T, int nw) {
  return static_cast<int>(((p + 1) * nw - 1) / T);
}

template <bool DEBUG>
__global__ __launch_bounds__(256) void protected_kernel(DecArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int wave = wave_id(), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int r16 = lane & 15, grp = lane >> 4;
  __shared__ __attribute__((aligned(16))) int8_t sv8[SIDE_ROWS][HD];  // INT8 V rows
  __shared__ float sz[GQA][SIDE_ROWS];                                // logits, then weights
  __shared__ float ssv[SIDE_ROWS];                                    // V scales

  const int h = g * GQA + wave;
  const size_t bh = static_cast<size_t>(b) * a.Hq + h;
  const int L = ld_const(a.ctx + b);
  const int slot = a.slot ? ld_const(a.slot + b) : b;
  const size_t row0 = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS;
  const gptr side = (gptr)a.side_codes + row0 * 2 * HD;
  const uint16_t* scales = a.side_scales + row0 * 2;

  // V rows straight into LDS: each wave instruction moves 8 rows (1 KB).
  for (int i = wave; i < SIDE_ROWS / 8; i += 4) {
    const int r = 8 * i + (lane >> 3);
    __builtin_amdgcn_global_load_lds(side + (2 * r + 1) * HD + 16 * (lane & 7),
                                     (lptr)(&sv8[8 * i][0]), 16, 0, 0);
  }
  for (int r = tid; r < SIDE_ROWS; r += 256)  // rows not in use: 0 (their weight is 0 too)
    ssv[r] = side_position(r, L) >= 0 ? f16_value(scales[2 * r + 1]) : 0.0f;

  // Main partials of this head, fetched now so their latency overlaps the
  // protected region (lane -> channels 2l, 2l+1).
  const int pb = ld_const(a.ws.plan + b);
  const int mp = (ld_const(a.ws.plan + b + 1) - pb) / a.Hkv;
  const int64_t T = ld_const(a.ws.plan + a.B);
  const int nw = a.ws.n_waves;
  int c_lo = 0, c_hi = -1;
  if (mp > 0) {
    const int64_t s0 = pb + static_cast<int64_t>(g) * mp;
    c_lo = chunk_of(s0, T, nw);
    c_hi = chunk_of(s0 + mp - 1, T, nw);
  }
  const size_t bg = static_cast<size_t>(b) * a.Hkv + g;
  constexpr int kBatch = 4;  // main partials fetched together
  float Zc[kBatch], lc[kBatch];
  float2 Ac[kBatch];
  bool okc[kBatch];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + i;
      okc[i] = (c <= c_hi) && (static_cast<int64_t>(c) * T / nw < static_cast<int64_t>(c + 1) * T / nw);
      const float* Pc = a.ws.parts + ((static_cast<size_t>(okc[i] ? c : 0) + bg) * GQA + wave) * kPart;
      Zc[i] = okc[i] ? Pc[128] : -INFINITY;
      lc[i] = okc[i] ? Pc[129] : 0.0f;
      Ac[i] = okc[i] ? reinterpret_cast<const float2*>(Pc)[lane] : make_float2(0.0f, 0.0f);
    }
  };
  fetch(c_lo);

  // INT8 QK on MFMA, 16 side rows per step; A = the 4 query codes (natural order).
  v4i qa[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (r16 < GQA) {
    const int8_t* qn = a.ws.qcodes + (static_cast<size_t>(b) * a.Hq + g * GQA + r16) * kQStride + HD;
    qa[0] = *reinterpret_cast<const v4i*>(qn + 16 * grp);
    qa[1] = *reinterpret_cast<const v4i*>(qn + 64 + 16 * grp);
  }
  const float c_q = ld_const(a.ws.qinfo + (static_cast<size_t>(b) * a.Hq + g * GQA + grp) * 4);
  for (int rg = wave; rg < SIDE_ROWS / 16; rg += 4) {
    const int r = 16 * rg + r16;
    const gptr krow = side + r * 2 * HD;
    v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(
        qa[0], *reinterpret_cast<const __attribute__((address_space(1))) v4i*>(krow + 16 * grp),
        v4i{0, 0, 0, 0}, 0, 0, 0);
    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(
        qa[1], *reinterpret_cast<const __attribute__((address_space(1))) v4i*>(krow + 64 + 16 * grp),
        d, 0, 0, 0);
    const int D8 = qk_rows(d);  // lane: head grp, row r
    const int p = side_position(r, L);
    const float sk = f16_value(scales[2 * r]);
    sz[grp][r] = (p >= 0) ? (static_cast<float>(D8) * sk) * c_q : -INFINITY;
    if (DEBUG && a.dbg.qk && p >= 0)
      a.dbg.qk[(static_cast<size_t>(b) * a.Hq + g * GQA + grp) * a.dbg.max_ctx + p] = D8;
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // V rows are in LDS
  __syncthreads();

  // FP32 softmax of this wave's head over the region (rows not in use: 0).
  float zl = -INFINITY;
  for (int i = lane; i < SIDE_ROWS; i += 64) zl = fmaxf(zl, sz[wave][i]);
  const float Z = wave_max(zl);
  float ls = 0.0f;
  for (int i = lane; i < SIDE_ROWS; i += 64) {
    const float e = exp2s(sz[wave][i] - Z);
    sz[wave][i] = e;
    ls += e;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // PV with BF16-dequantized values v^ = bf16(s_v c) and FP32 weights.
  float a0 = 0.0f, a1 = 0.0f;
  for (int r = 0; r < SIDE_ROWS; r += 4) {
    const float4 e4 = *reinterpret_cast<const float4*>(&sz[wave][r]);
    const float4 s4 = *reinterpret_cast<const float4*>(&ssv[r]);
    const float ev[4] = {e4.x, e4.y, e4.z, e4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t cc = reinterpret_cast<const uint16_t*>(sv8[r + i])[lane];
      const float v0 = round_bf16(sv[i] * static_cast<float>(static_cast<int8_t>(cc & 0xFF)));
      const float v1 = round_bf16(sv[i] * static_cast<float>(static_cast<int8_t>(cc >> 8)));
      a0 = __builtin_fmaf(ev[i], v0, a0);
      a1 = __builtin_fmaf(ev[i], v1, a1);
    }
  }
  // exact log-sum-exp merge with the main partials of this head
  float Zm = Z, lm = ls;
  float2 Am = make_float2(a0, a1);
  for (int c0 = c_lo; c0 <= c_hi; c0 += kBatch) {
    if (c0 != c_lo) fetch(c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (!okc[i]) continue;
      const float Zn = fmaxf(Zm, Zc[i]);
      const float w0 = __builtin_amdgcn_exp2f(Zm - Zn), w1 = __builtin_amdgcn_exp2f(Zc[i] - Zn);
      Am.x = Am.x * w0 + Ac[i].x * w1;
      Am.y = Am.y * w0 + Ac[i].y * w1;
      lm = lm * w0 + lc[i] * w1;
      Zm = Zn;
    }
  }
  reinterpret_cast<float2*>(a.out + bh * HD)[lane] = make_float2(Am.x / lm, Am.y / lm);
  if (lane == 0) a.lse[bh] = 0.69314718055994531f * (Zm + log2f(lm));
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int n_waves) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t n = up(static_cast<size_t>(B + 1) * 4);
  n += up(static_cast<size_t>(B) * Hq * kQStride);
  n += up(static_cast<size_t>(B) * Hq * 4 * 4);
  n += up((static_cast<size_t>(n_waves) + static_cast<size_t>(B) * Hkv) * GQA * kPart * 4);
  return n;
}

DecodeWorkspace carve_workspace(void* base, int B, int Hq, int Hkv, int n_waves) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  char* p = static_cast<char*>(base);
  DecodeWorkspace w;
  w.plan = reinterpret_cast<int32_t*>(p);
  p += up(static_cast<size_t>(B + 1) * 4);
  w.qcodes = reinterpret_cast<int8_t*>(p);
  p += up(static_cast<size_t>(B) * Hq * kQStride);
  w.qinfo = reinterpret_cast<float*>(p);
  p += up(static_cast<size_t>(B) * Hq * 4 * 4);
  w.parts = reinterpret_cast<float*>(p);
  w.n_waves = n_waves;
  return w;
}

hipError_t launch_decode(const CacheView& c, const uint16_t* q, const int32_t* ctx,
                         const int32_t* slot, const int32_t* page_table, int pt_stride, int B,
                         int Hq, float scale_log2, float* out, float* lse,
                         const DecodeWorkspace& ws, const DecodeDebug* dbg, hipStream_t s,
                         hipEvent_t ev_main_begin, hipEvent_t ev_main_end) {
  DecArgs a{};
  a.pages = c.pages;
  a.side_codes = c.side_codes;
  a.side_scales = c.side_scales;
  a.Hkv = c.Hkv;
  a.Hq = Hq;
  a.B = B;
  a.q = reinterpret_cast<const uint32_t*>(q);
  a.ctx = ctx;
  a.slot = slot;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.scale_log2 = scale_log2;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  if (dbg) a.dbg = *dbg;
  const dim3 block(256), groups(c.Hkv, B), grid(ws.n_waves / 4);
  if (dbg) {
    hipLaunchKernelGGL(query_kernel<true>, groups, block, 0, s, a);
    hipLaunchKernelGGL(main_kernel<true>, grid, block, 0, s, a);
    hipLaunchKernelGGL(protected_kernel<true>, groups, block, 0, s, a);
  } else {
    hipLaunchKernelGGL(query_kernel<false>, groups, block, 0, s, a);
    if (ev_main_begin) {
      const hipError_t e = hipEventRecord(ev_main_begin, s);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(main_kernel<false>, grid, block, 0, s, a);
    if (ev_main_end) {
      const hipError_t e = hipEventRecord(ev_main_end, s);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(protected_kernel<false>, groups, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kv4
