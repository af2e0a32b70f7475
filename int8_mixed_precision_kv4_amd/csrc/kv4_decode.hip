// kv4_decode.hip -- one decode step of KV4-RL hybrid attention
// (paper.rainbus.top summary, "方法步骤详情" step 4 and "核心方法"; onedev.kr
// summary, "전제와 한계").
//
// Three launches on the caller's stream:
//   1. protected_kernel, one workgroup per (kv-head, sequence): rotates and
//      INT8-quantizes the 4 queries of the group (the codes are reused by the
//      main region), runs INT8 QK against the side keys, an FP32 softmax, and
//      PV over BF16-dequantized side values.  Workgroup (0,0) also writes the
//      main-region work plan (prefix sums of main pages).
//   2. main_kernel, a fixed grid of independent waves: the concatenated list
//      of main-region pages of all (sequence, kv-head) pairs is cut into equal
//      contiguous chunks, one per wave (split-K with exact load balance).  Per
//      page: integer QK on MFMA (INT8 query x unpacked INT4 keys), delta/m
//      applied after the dot, tile softmax, INT8 P operand with the V scale
//      folded in, integer PV on MFMA, FP32 running merge.  A wave writes one
//      partial per (sequence, kv-head) segment it touches.
//   3. merge_kernel, one wave per (sequence, q-head): exact log-sum-exp merge
//      of the protected partial and the main partials.
#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace kv4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ int side_row(int p) { return p < SINK ? p : SINK + (p % WINDOW); }

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

// ------------------------------------------------------------- protected --

template <bool DEBUG>
__global__ __launch_bounds__(256) void protected_kernel(DecArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
  if (g == 0 && b == 0) build_plan(a);

  __shared__ int32_t sq[GQA][HD / 4];      // query codes, 4 per dword, natural order
  __shared__ float scq[GQA];
  __shared__ float sz[GQA][SIDE_ROWS];     // logits, then weights
  __shared__ int32_t sv8[SIDE_ROWS][HD / 4];
  __shared__ float ssv[SIDE_ROWS];

  const int h = g * GQA + wave;
  const size_t bh = static_cast<size_t>(b) * a.Hq + h;
  const int L = a.ctx[b];
  const int slot = a.slot ? a.slot[b] : b;

  // Rotate the query like the keys, then symmetric INT8 with an FP32 scale.
  {
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
    const float c_q = s_q * a.scale_log2;
    reinterpret_cast<uint16_t*>(sq[wave])[lane] =
        static_cast<uint16_t>((c0 & 0xFF) | ((c1 & 0xFF) << 8));
    // even channels then odd channels, the operand order of the main kernel
    int8_t* qs = a.ws.qcodes + bh * HD;
    qs[lane] = static_cast<int8_t>(c0);
    qs[64 + lane] = static_cast<int8_t>(c1);
    if (lane == 0) {
      a.ws.qinfo[bh * 4 + 0] = c_q;
      a.ws.qinfo[bh * 4 + 1] = __int_as_float(S);
      a.ws.qinfo[bh * 4 + 2] = s_q;
      a.ws.qinfo[bh * 4 + 3] = 0.0f;
      scq[wave] = c_q;
      if (DEBUG && a.dbg.qsum) a.dbg.qsum[bh] = S;
    }
    if (DEBUG && a.dbg.qcodes) {
      a.dbg.qcodes[bh * HD + 2 * lane] = static_cast<int8_t>(c0);
      a.dbg.qcodes[bh * HD + 2 * lane + 1] = static_cast<int8_t>(c1);
    }
  }
  __syncthreads();

  // Protected positions: sinks [0, min(16,L)) then recent [max(16,L-128), L).
  const int n = min(L, SIDE_ROWS);
  const int sink_end = min(SINK, L), rec_begin = max(SINK, L - WINDOW);
  if (tid < n) {
    const int p = tid < sink_end ? tid : rec_begin + (tid - sink_end);
    const size_t r = (static_cast<size_t>(slot) * a.Hkv + g) * SIDE_ROWS + side_row(p);
    const int4* krow = reinterpret_cast<const int4*>(a.side_codes + r * 2 * HD);
    const int4* vrow = krow + HD / 16;
    int d[GQA] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      const int4 kk = krow[c];
      const int4 vv = vrow[c];
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        d[hh] = __builtin_amdgcn_sdot4(kk.x, sq[hh][4 * c + 0], d[hh], false);
        d[hh] = __builtin_amdgcn_sdot4(kk.y, sq[hh][4 * c + 1], d[hh], false);
        d[hh] = __builtin_amdgcn_sdot4(kk.z, sq[hh][4 * c + 2], d[hh], false);
        d[hh] = __builtin_amdgcn_sdot4(kk.w, sq[hh][4 * c + 3], d[hh], false);
      }
      sv8[tid][4 * c + 0] = vv.x;
      sv8[tid][4 * c + 1] = vv.y;
      sv8[tid][4 * c + 2] = vv.z;
      sv8[tid][4 * c + 3] = vv.w;
    }
    const float sk = f16_value(a.side_scales[r * 2 + 0]);
    ssv[tid] = f16_value(a.side_scales[r * 2 + 1]);
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      sz[hh][tid] = (static_cast<float>(d[hh]) * sk) * scq[hh];
      if (DEBUG && a.dbg.qk)
        a.dbg.qk[(static_cast<size_t>(b) * a.Hq + g * GQA + hh) * a.dbg.max_ctx + p] = d[hh];
    }
  }
  __syncthreads();

  // FP32 softmax of this wave's head over the region.
  float zl = -INFINITY;
  for (int i = lane; i < n; i += 64) zl = fmaxf(zl, sz[wave][i]);
  const float Z = wave_max(zl);
  float ls = 0.0f;
  for (int i = lane; i < n; i += 64) {
    const float e = exp2s(sz[wave][i] - Z);
    sz[wave][i] = e;
    ls += e;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
  __syncthreads();

  // PV with BF16-dequantized values, P kept in FP32; lane -> channels 2l, 2l+1.
  float a0 = 0.0f, a1 = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float e = sz[wave][i];
    const float sv = ssv[i];
    const uint32_t cc = reinterpret_cast<const uint16_t*>(sv8[i])[lane];
    const float v0 = round_bf16(sv * static_cast<float>(static_cast<int8_t>(cc & 0xFF)));
    const float v1 = round_bf16(sv * static_cast<float>(static_cast<int8_t>(cc >> 8)));
    a0 = __builtin_fmaf(e, v0, a0);
    a1 = __builtin_fmaf(e, v1, a1);
  }
  float* P = a.ws.prot + bh * kPart;
  reinterpret_cast<float2*>(P)[lane] = make_float2(a0, a1);
  if (lane == 0) {
    P[128] = Z;
    P[129] = ls;
  }
}

// ------------------------------------------------------------------ main --

__device__ __forceinline__ v4i nib_lo(uint4 x) {
  const uint32_t m = 0x0F0F0F0Fu;
  return v4i{static_cast<int>(x.x & m), static_cast<int>(x.y & m), static_cast<int>(x.z & m),
             static_cast<int>(x.w & m)};
}
__device__ __forceinline__ v4i nib_hi(uint4 x) {
  const uint32_t m = 0x0F0F0F0Fu;
  return v4i{static_cast<int>((x.x >> 4) & m), static_cast<int>((x.y >> 4) & m),
             static_cast<int>((x.z >> 4) & m), static_cast<int>((x.w >> 4) & m)};
}
// 16 positions of one channel (8 nibble bytes) -> 16 INT8 operand bytes; byte
// i of the result holds position 8(i/8) + 2(i%4) + (i/4)%2.
__device__ __forceinline__ v4i nib_positions(uint32_t lo8, uint32_t hi8) {
  const uint32_t m = 0x0F0F0F0Fu;
  return v4i{static_cast<int>(lo8 & m), static_cast<int>((lo8 >> 4) & m),
             static_cast<int>(hi8 & m), static_cast<int>((hi8 >> 4) & m)};
}
// inverse of that byte order
__device__ __forceinline__ int pcode_slot(int t) { return 8 * (t >> 3) + 4 * (t & 1) + ((t & 7) >> 1); }

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

template <bool DEBUG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void main_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t pstage[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * 4 + wave;
  const int nw = a.ws.n_waves;
  const int32_t* plan = a.ws.plan;
  const int64_t T = plan[a.B];
  const int64_t start = static_cast<int64_t>(w) * T / nw;
  const int64_t end = static_cast<int64_t>(w + 1) * T / nw;
  if (start >= end) return;
  int lo = 0, hi = a.B;  // plan[lo] <= start < plan[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (plan[mid] <= start) lo = mid;
    else hi = mid;
  }
  int b = lo;
  uint8_t* stage = pstage[wave];
  int64_t page = start;

  while (page < end) {
    while (plan[b + 1] <= page) ++b;
    const int mp = (plan[b + 1] - plan[b]) / a.Hkv;
    const int g = static_cast<int>((page - plan[b]) / mp);
    const int64_t seg0 = plan[b] + static_cast<int64_t>(g) * mp;
    const int64_t stop = min(end, seg0 + mp);
    const int main_end = a.ctx[b] - WINDOW;
    const size_t qb = static_cast<size_t>(b) * a.Hq + g * GQA;

    // A operand of QK: rows 0..3 = the group's heads, k = channels
    // (lane group grp covers channels 32grp..32grp+31, even / odd split).
    v4i qa0 = {0, 0, 0, 0}, qa1 = {0, 0, 0, 0};
    if (r16 < GQA) {
      const int8_t* qs = a.ws.qcodes + (qb + r16) * HD;
      qa0 = *reinterpret_cast<const v4i*>(qs + 16 * grp);
      qa1 = *reinterpret_cast<const v4i*>(qs + 64 + 16 * grp);
    }
    const float c_q = a.ws.qinfo[(qb + grp) * 4 + 0];
    const float S_q = static_cast<float>(__float_as_int(a.ws.qinfo[(qb + grp) * 4 + 1]));

    float Zr = -INFINITY, Ls = 0.0f, Ms = 0.0f;
    float O[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int32_t* ptrow = a.page_table + static_cast<size_t>(b) * a.pt_stride;

    for (int64_t p0 = page; p0 < stop; p0 += 4) {
      const int np = static_cast<int>(min(static_cast<int64_t>(4), stop - p0));
      const int j0 = 1 + static_cast<int>(p0 - seg0);  // logical page of tile 0
      const uint8_t* blk[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int phys = ptrow[j0 + min(t, np - 1)];
        blk[t] = a.pages + (static_cast<size_t>(phys) * a.Hkv + g) * BLOCK_BYTES;
      }
      uint4 kq[4], vq[4];
      uint32_t km[4], vm[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        kq[t] = *reinterpret_cast<const uint4*>(blk[t] + 64 * r16 + 16 * grp);
        km[t] = *reinterpret_cast<const uint32_t*>(blk[t] + OFF_KMETA + 4 * r16);
        vm[t] = *reinterpret_cast<const uint32_t*>(blk[t] + OFF_VMETA + 4 * r16);
      }
      const uint8_t* vb = grp == 0 ? blk[0] : grp == 1 ? blk[1] : grp == 2 ? blk[2] : blk[3];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        vq[s2] = *reinterpret_cast<const uint4*>(vb + OFF_VCODE + 16 * (16 * s2 + r16));

      float zmax[4], su[4], ecol[4], emv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa0, nib_lo(kq[t]), v4i{0, 0, 0, 0}, 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa1, nib_hi(kq[t]), d, 0, 0, 0);
        const int D = qk_rows(d);  // lane: head grp, position r16 of tile t
        const int pos = PAGE * (j0 + t) + r16;
        const bool valid = (t < np) && (pos < main_end);
        const float dk = f16_value(km[t] & 0xFFFFu), mk = f16_value(km[t] >> 16);
        const float dv = f16_value(vm[t] & 0xFFFFu), mv = f16_value(vm[t] >> 16);
        // q.k^ = s_q (delta * sum(qc*c) + m * sum(qc)); c_q carries s_q, the scale and log2(e)
        float z = __builtin_fmaf(dk, static_cast<float>(D), mk * S_q) * c_q;
        z = valid ? z : -INFINITY;
        zmax[t] = row16_max(z);
        const float e = valid ? exp2s(z - zmax[t]) : 0.0f;
        const float u = valid ? e * dv : 0.0f;  // V scale folded into P
        const float umax = row16_max(u);
        uint32_t uc = 0;
        if (umax != 0.0f) {
          const float inv = 127.0f / umax;
          uc = static_cast<uint32_t>(fminf(fmaxf(__builtin_rintf(u * inv), 0.0f), 127.0f));
        }
        su[t] = umax * (1.0f / 127.0f);
        ecol[t] = e;
        emv[t] = valid ? e * mv : 0.0f;  // V offset applied after the dot
        stage[(t * 4 + grp) * 16 + pcode_slot(r16)] = static_cast<uint8_t>(uc);
        if (DEBUG && valid) {
          const size_t row = (qb + grp) * a.dbg.max_ctx + pos;
          if (a.dbg.qk) a.dbg.qk[row] = D;
          if (a.dbg.pcode) a.dbg.pcode[row] = static_cast<uint8_t>(uc);
        }
      }
      // running reference max of each head; rescale what is accumulated
      const float Zn = fmaxf(Zr, fmaxf(fmaxf(zmax[0], zmax[1]), fmaxf(zmax[2], zmax[3])));
      const float al = __builtin_amdgcn_exp2f(Zr - Zn);
#pragma unroll
      for (int o = 0; o < 8; ++o) O[o] *= al;
      Ls *= al;
      Ms *= al;
      Zr = Zn;
      float wsu[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float wt = __builtin_amdgcn_exp2f(zmax[t] - Zr);
        Ls = __builtin_fmaf(wt, ecol[t], Ls);
        Ms = __builtin_fmaf(wt, emv[t], Ms);
        wsu[t] = wt * su[t];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // A operand of PV: row 4h + tau, k-group = tile; block diagonal in tiles
      v4i pa = *reinterpret_cast<const v4i*>(stage + (grp * 4 + (r16 >> 2)) * 16);
      if ((r16 & 3) != grp) pa = v4i{0, 0, 0, 0};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const v4i bv = e2 == 0 ? nib_positions(vq[s2].x, vq[s2].y) : nib_positions(vq[s2].z, vq[s2].w);
          const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa, bv, v4i{0, 0, 0, 0}, 0, 0, 0);
          // lane: head grp, channel 2(16 s2 + r16) + e2, tile v in register v
          float o = O[2 * s2 + e2];
          o = __builtin_fmaf(wsu[0], static_cast<float>(acc[0]), o);
          o = __builtin_fmaf(wsu[1], static_cast<float>(acc[1]), o);
          o = __builtin_fmaf(wsu[2], static_cast<float>(acc[2]), o);
          o = __builtin_fmaf(wsu[3], static_cast<float>(acc[3]), o);
          O[2 * s2 + e2] = o;
          if (DEBUG && a.dbg.pv) {
            const int ch = 2 * (16 * s2 + r16) + e2;
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (t < np)
                a.dbg.pv[((qb + grp) * a.dbg.max_pages + (j0 + t)) * HD + ch] = acc[t];
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // partial of this (sequence, kv-head) segment: A = O + sum(w e m_v)
    const float Lh = row16_sum(Ls), Mh = row16_sum(Ms);
    float* P = a.ws.parts + ((static_cast<size_t>(w) + static_cast<size_t>(b) * a.Hkv + g) * GQA + grp) * kPart;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      *reinterpret_cast<float2*>(P + 2 * (16 * s2 + r16)) = make_float2(O[2 * s2] + Mh, O[2 * s2 + 1] + Mh);
    if (r16 == 0) {
      P[128] = Zr;
      P[129] = Lh;
    }
    page = stop;
  }
}

// ----------------------------------------------------------------- merge --

__global__ __launch_bounds__(256) void merge_kernel(DecArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave, b = blockIdx.y;
  if (h >= a.Hq) return;
  const int g = h / GQA, hh = h % GQA;
  const size_t bh = static_cast<size_t>(b) * a.Hq + h;
  const float* P0 = a.ws.prot + bh * kPart;
  float Z = P0[128], l = P0[129];
  float2 A = reinterpret_cast<const float2*>(P0)[lane];
  const int32_t* plan = a.ws.plan;
  const int64_t T = plan[a.B];
  const int mp = (plan[b + 1] - plan[b]) / a.Hkv;
  if (mp > 0) {
    const int nw = a.ws.n_waves;
    const int64_t s = plan[b] + static_cast<int64_t>(g) * mp, e = s + mp;
    const int c_lo = static_cast<int>(((s + 1) * nw - 1) / T);
    const int c_hi = static_cast<int>((e * nw - 1) / T);
    for (int c = c_lo; c <= c_hi; ++c) {
      if (static_cast<int64_t>(c) * T / nw >= static_cast<int64_t>(c + 1) * T / nw) continue;
      const float* Pc = a.ws.parts + ((static_cast<size_t>(c) + static_cast<size_t>(b) * a.Hkv + g) * GQA + hh) * kPart;
      const float Zc = Pc[128], lc = Pc[129];
      const float2 Ac = reinterpret_cast<const float2*>(Pc)[lane];
      const float Zn = fmaxf(Z, Zc);
      const float w0 = __builtin_amdgcn_exp2f(Z - Zn), w1 = __builtin_amdgcn_exp2f(Zc - Zn);
      A.x = A.x * w0 + Ac.x * w1;
      A.y = A.y * w0 + Ac.y * w1;
      l = l * w0 + lc * w1;
      Z = Zn;
    }
  }
  reinterpret_cast<float2*>(a.out + bh * HD)[lane] = make_float2(A.x / l, A.y / l);
  if (lane == 0) a.lse[bh] = 0.69314718055994531f * (Z + log2f(l));
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int n_waves) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t n = up(static_cast<size_t>(B + 1) * 4);
  n += up(static_cast<size_t>(B) * Hq * HD);
  n += up(static_cast<size_t>(B) * Hq * 4 * 4);
  n += up(static_cast<size_t>(B) * Hq * kPart * 4);
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
  p += up(static_cast<size_t>(B) * Hq * HD);
  w.qinfo = reinterpret_cast<float*>(p);
  p += up(static_cast<size_t>(B) * Hq * 4 * 4);
  w.prot = reinterpret_cast<float*>(p);
  p += up(static_cast<size_t>(B) * Hq * kPart * 4);
  w.parts = reinterpret_cast<float*>(p);
  w.n_waves = n_waves;
  return w;
}

hipError_t launch_decode(const CacheView& c, const uint16_t* q, const int32_t* ctx,
                         const int32_t* slot, const int32_t* page_table, int pt_stride, int B,
                         int Hq, float scale_log2, float* out, float* lse,
                         const DecodeWorkspace& ws, const DecodeDebug* dbg, hipStream_t s) {
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
  const dim3 block(256);
  if (dbg) {
    hipLaunchKernelGGL(protected_kernel<true>, dim3(c.Hkv, B), block, 0, s, a);
    hipLaunchKernelGGL(main_kernel<true>, dim3(ws.n_waves / 4), block, 0, s, a);
  } else {
    hipLaunchKernelGGL(protected_kernel<false>, dim3(c.Hkv, B), block, 0, s, a);
    hipLaunchKernelGGL(main_kernel<false>, dim3(ws.n_waves / 4), block, 0, s, a);
  }
  hipLaunchKernelGGL(merge_kernel, dim3((Hq + 3) / 4, B), block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kv4
