// prefill_f32.hip - the same attention as prefill_bf16.hip with fp32 inputs,
// fp32 outputs and fp32 arithmetic throughout (no bf16 rounding anywhere).
//
// It follows the tiled recurrence of the "Real-time inference optimisation"
// page (section "Flash Attention optimisation"): per row a running max, a
// running sum and a rescaled accumulator over K/V tiles held on chip. The fp32
// path serves small, launch-latency-bound shapes, so it uses the vector ALU
// (CDNA4 has no fp32 MFMA rate worth trading accuracy for) and accurate expf.
//
// Work-group: 256 threads own 64 query rows, 4 threads per row; each thread
// holds D/4 consecutive dims of its row's q and of its output accumulator.
// A dot product is a per-thread partial sum plus a 2-step reduction across the
// 4 threads of the row (DPP quad permutes). K/V tiles of 32 rows sit in LDS and
// every thread reads them as broadcast float4s.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRows = 64;  // query rows per work-group
constexpr int kKT = 32;    // keys per LDS tile

__device__ __forceinline__ float quad_sum(float x) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of the quad ends with the sum.
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  return x;
}

template <int D>
__global__ void __launch_bounds__(256) prefill_f32_kernel(PrefillParams p, float scale) {
  constexpr int DP = D / 4;  // dims per thread
  __shared__ __attribute__((aligned(16))) float sK[kKT * D];
  __shared__ __attribute__((aligned(16))) float sV[kKT * D];

  const int tid = threadIdx.x;
  const int rl = tid >> 2, part = tid & 3;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq, Skv = p.Skv, off = Skv - Sq;
  const bool causal = p.causal != 0;
  const int row = qt * kRows + rl;
  const bool valid = row < Sq;

  float q[DP], acc[DP];
  const float* qrow = (const float*)p.q + (((size_t)b * p.Hq + h) * Sq + (valid ? row : 0)) * D + part * DP;
#pragma unroll
  for (int e = 0; e < DP; e += 4) {
    float4 x = valid ? *(const float4*)(qrow + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = x.x; q[e + 1] = x.y; q[e + 2] = x.z; q[e + 3] = x.w;
  }
#pragma unroll
  for (int e = 0; e < DP; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last_row = min(Sq, (qt + 1) * kRows) - 1;
  const int kend = causal ? min(Skv, last_row + off + 1) : Skv;  // keys this work-group needs
  const int lim = causal ? row + off : Skv - 1;                    // last key visible to this row
  const float* kbh = (const float*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const float* vbh = (const float*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;

  for (int k0 = 0; k0 < kend; k0 += kKT) {
    __syncthreads();
    // cooperative tile load: kKT*D floats as float4, rows past Skv clamped
    for (int f = tid; f < kKT * D / 4; f += 256) {
      const int r = (f * 4) / D, cidx = (f * 4) % D;
      const int gr = min(k0 + r, Skv - 1);
      *(float4*)(sK + r * D + cidx) = *(const float4*)(kbh + (size_t)gr * D + cidx);
      *(float4*)(sV + r * D + cidx) = *(const float4*)(vbh + (size_t)gr * D + cidx);
    }
    __syncthreads();
    float s[kKT];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kKT; ++jj) {
      const float* kr = sK + jj * D + part * DP;
      float sp = 0.f;
#pragma unroll
      for (int e = 0; e < DP; e += 4) {
        const float4 x = *(const float4*)(kr + e);
        sp = fmaf(q[e], x.x, sp);
        sp = fmaf(q[e + 1], x.y, sp);
        sp = fmaf(q[e + 2], x.z, sp);
        sp = fmaf(q[e + 3], x.w, sp);
      }
      sp = quad_sum(sp) * scale;
      const int key = k0 + jj;
      s[jj] = (key <= lim && key < Skv) ? sp : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) acc[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kKT; ++jj) {
      const float pj = (s[jj] == -INFINITY) ? 0.f : expf(s[jj] - mu);
      l += pj;
      const float* vr = sV + jj * D + part * DP;
#pragma unroll
      for (int e = 0; e < DP; e += 4) {
        const float4 x = *(const float4*)(vr + e);
        acc[e] = fmaf(pj, x.x, acc[e]);
        acc[e + 1] = fmaf(pj, x.y, acc[e + 1]);
        acc[e + 2] = fmaf(pj, x.z, acc[e + 2]);
        acc[e + 3] = fmaf(pj, x.w, acc[e + 3]);
      }
    }
    m = mn;
  }
  if (valid) {
    const float inv = 1.0f / l;
    float* orow = (float*)p.o + (((size_t)b * p.Hq + h) * Sq + row) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; e += 4)
      *(float4*)(orow + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, int d, float scale, hipStream_t stream) {
  dim3 grid((p.Sq + kRows - 1) / kRows, p.Hq, p.B), block(256);
  if (d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, stream, p, scale);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, stream, p, scale);
  return hipGetLastError();
}

}  // namespace fa
