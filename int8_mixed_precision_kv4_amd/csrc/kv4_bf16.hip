// kv4_bf16.hip -- comparator: ordinary BF16 paged decode attention (the
// baseline the KV4-RL pages measure their speed-ups against), written with the
// same work decomposition as the KV4 main region so the two are timed on equal
// terms: a plan of page prefix sums, equal contiguous page chunks per wave,
// QK and PV on BF16 MFMA with FP32 accumulation, and an exact log-sum-exp merge.
// Its page loads are non-temporal like the KV4 kernel's (each page is read once).
//
// Pool layout bf16 [num_pages][Hkv][2][16][128]: per (page, kv-head) the K
// block is token-major [16 positions][128 channels] and the V block is
// channel-major [128 channels][16 positions].
#include "kv4_device.hpp"
#include "kv4_internal.hpp"

namespace kv4 {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBlock16 = 2 * PAGE * HD;  // bf16 elements per (page, kv-head)

struct BfArgs {
  const uint16_t* pages;
  int Hkv, Hq, B;
  const uint16_t* q;
  const int32_t* ctx;
  const int32_t* page_table;
  int pt_stride;
  float scale_log2;
  float* out;
  float* lse;
  int32_t* plan;  // [B+1]
  float* parts;   // [n_waves + B*Hkv][4][kPart]
  int n_waves;
};

__global__ __launch_bounds__(256) void bf16_plan_kernel(BfArgs a) {
  __shared__ int32_t scan[256];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) {
    carry = 0;
    a.plan[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < a.B; base += 256) {
    const int b = base + threadIdx.x;
    scan[threadIdx.x] = (b < a.B) ? ((a.ctx[b] + PAGE - 1) / PAGE) * a.Hkv : 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int t = (threadIdx.x >= off) ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += t;
      __syncthreads();
    }
    if (b < a.B) a.plan[b + 1] = carry + scan[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 255) carry += scan[255];
    __syncthreads();
  }
}

// QK output with each head's query in four A rows (row r = head r / 4): lane
// l holds head l / 16 at position l % 16 in every register.
__device__ __forceinline__ float qk_rows_f(v4f d) { return d[0]; }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void bf16_main_kernel(BfArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 pstage[4][GQA][2 * PAGE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * 4 + wave;
  const int nw = a.n_waves;
  const int64_t T = a.plan[a.B];
  const int64_t start = static_cast<int64_t>(w) * T / nw;
  const int64_t end = static_cast<int64_t>(w + 1) * T / nw;
  if (start >= end) return;
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.plan[mid] <= start) lo = mid;
    else hi = mid;
  }
  int b = lo;
  int64_t page = start;
  while (page < end) {
    while (a.plan[b + 1] <= page) ++b;
    const int np_seq = (a.plan[b + 1] - a.plan[b]) / a.Hkv;
    const int g = static_cast<int>((page - a.plan[b]) / np_seq);
    const int64_t seg0 = a.plan[b] + static_cast<int64_t>(g) * np_seq;
    const int64_t stop = min(end, seg0 + np_seq);
    const int L = a.ctx[b];
    const size_t qb = static_cast<size_t>(b) * a.Hq + g * GQA;
    v8bf qa[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      qa[m] = *reinterpret_cast<const v8bf*>(a.q + (qb + (r16 >> 2)) * HD + 32 * m + 8 * grp);
    float Zr = -INFINITY, Ls = 0.0f;
    v4f O[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) O[s] = v4f{0, 0, 0, 0};
    const int32_t* ptrow = a.page_table + static_cast<size_t>(b) * a.pt_stride;

    for (int64_t p0 = page; p0 < stop; p0 += 2) {
      const int np = static_cast<int>(min(static_cast<int64_t>(2), stop - p0));
      const int j0 = static_cast<int>(p0 - seg0);
      const uint16_t* blk[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int phys = ptrow[j0 + min(t, np - 1)];
        blk[t] = a.pages + (static_cast<size_t>(phys) * a.Hkv + g) * kBlock16;
      }
      v8bf kb[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          kb[t][m] = __builtin_nontemporal_load(reinterpret_cast<const v8bf*>(blk[t] + r16 * HD + 32 * m + 8 * grp));
      // V: lane group grp covers positions 8grp..8grp+7 of the page pair
      const uint16_t* vblk = (grp < 2 ? blk[0] : blk[1]) + PAGE * HD + 8 * (grp & 1);
      v8bf vb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        vb[s] = __builtin_nontemporal_load(reinterpret_cast<const v8bf*>(vblk + (16 * s + r16) * PAGE));

      float z[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        v4f d = v4f{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 4; ++m) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[m], kb[t][m], d, 0, 0, 0);
        const float D = qk_rows_f(d);
        const int pos = PAGE * (j0 + t) + r16;
        z[t] = (t < np && pos < L) ? D * a.scale_log2 : -INFINITY;
      }
      const float Zn = fmaxf(Zr, fmaxf(row16_max(z[0]), row16_max(z[1])));
      const float al = __builtin_amdgcn_exp2f(Zr - Zn);
      Zr = Zn;
      const float p0v = __builtin_amdgcn_exp2f(z[0] - Zn), p1v = __builtin_amdgcn_exp2f(z[1] - Zn);
      Ls = Ls * al + p0v + p1v;
      pstage[wave][grp][r16] = static_cast<__bf16>(p0v);
      pstage[wave][grp][PAGE + r16] = static_cast<__bf16>(p1v);
      // the running rescale of O: head v lives in register v of lanes 0..15
      float alh[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) alh[v] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 16 * v));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      v8bf pa = v8bf{};
      if (r16 < GQA) pa = *reinterpret_cast<const v8bf*>(&pstage[wave][r16][8 * grp]);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        v4f o = O[s];
        o[0] *= alh[0];
        o[1] *= alh[1];
        o[2] *= alh[2];
        o[3] *= alh[3];
        O[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb[s], o, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    }
    const float Lh = row16_sum(Ls);
    float* P = a.parts + ((static_cast<size_t>(w) + static_cast<size_t>(b) * a.Hkv + g) * GQA) * kPart;
    if (grp == 0) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int v = 0; v < 4; ++v) P[v * kPart + 16 * s + r16] = O[s][v];
    }
    if (r16 == 0) {
      P[grp * kPart + 128] = Zr;
      P[grp * kPart + 129] = Lh;
    }
    page = stop;
  }
}

__global__ __launch_bounds__(256) void bf16_merge_kernel(BfArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave, b = blockIdx.y;
  if (h >= a.Hq) return;
  const int g = h / GQA, hh = h % GQA;
  const size_t bh = static_cast<size_t>(b) * a.Hq + h;
  float Z = -INFINITY, l = 0.0f;
  float2 A = make_float2(0.0f, 0.0f);
  const int64_t T = a.plan[a.B];
  const int np = (a.plan[b + 1] - a.plan[b]) / a.Hkv;
  const int nw = a.n_waves;
  const int64_t s = a.plan[b] + static_cast<int64_t>(g) * np, e = s + np;
  const int c_lo = static_cast<int>(((s + 1) * nw - 1) / T);
  const int c_hi = static_cast<int>((e * nw - 1) / T);
  for (int c = c_lo; c <= c_hi; ++c) {
    if (static_cast<int64_t>(c) * T / nw >= static_cast<int64_t>(c + 1) * T / nw) continue;
    const float* Pc = a.parts + ((static_cast<size_t>(c) + static_cast<size_t>(b) * a.Hkv + g) * GQA + hh) * kPart;
    const float Zc = Pc[128], lc = Pc[129];
    const float2 Ac = reinterpret_cast<const float2*>(Pc)[lane];
    const float Zn = fmaxf(Z, Zc);
    const float w0 = __builtin_amdgcn_exp2f(Z - Zn), w1 = __builtin_amdgcn_exp2f(Zc - Zn);
    A.x = A.x * w0 + Ac.x * w1;
    A.y = A.y * w0 + Ac.y * w1;
    l = l * w0 + lc * w1;
    Z = Zn;
  }
  reinterpret_cast<float2*>(a.out + bh * HD)[lane] = make_float2(A.x / l, A.y / l);
  if (lane == 0) a.lse[bh] = 0.69314718055994531f * (Z + log2f(l));
}

}  // namespace

size_t bf16_workspace_bytes(int B, int Hq, int Hkv, int n_waves) {
  (void)Hq;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return up(static_cast<size_t>(B + 1) * 4) +
         up((static_cast<size_t>(n_waves) + static_cast<size_t>(B) * Hkv) * GQA * kPart * 4);
}

hipError_t launch_bf16_decode(const uint16_t* pages, int num_pages, int Hkv, const uint16_t* q,
                              const int32_t* ctx, const int32_t* page_table, int pt_stride, int B,
                              int Hq, float scale_log2, float* out, float* lse, void* ws,
                              int n_waves, hipStream_t s) {
  (void)num_pages;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  BfArgs a{};
  a.pages = pages;
  a.Hkv = Hkv;
  a.Hq = Hq;
  a.B = B;
  a.q = q;
  a.ctx = ctx;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.scale_log2 = scale_log2;
  a.out = out;
  a.lse = lse;
  a.plan = static_cast<int32_t*>(ws);
  a.parts = reinterpret_cast<float*>(static_cast<char*>(ws) + up(static_cast<size_t>(B + 1) * 4));
  a.n_waves = n_waves;
  hipLaunchKernelGGL(bf16_plan_kernel, dim3(1), dim3(256), 0, s, a);
  hipLaunchKernelGGL(bf16_main_kernel, dim3(n_waves / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(bf16_merge_kernel, dim3((Hq + 3) / 4, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kv4
