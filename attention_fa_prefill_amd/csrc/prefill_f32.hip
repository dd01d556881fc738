// prefill_f32.hip - the same attention as prefill_bf16.hip with fp32 inputs,
// fp32 outputs and fp32 arithmetic throughout (no bf16 rounding anywhere).
//
// It follows the tiled recurrence of the "Real-time inference optimisation"
// page (section "Flash Attention optimisation"): per row a running max, a
// running sum and a rescaled accumulator over blocks of keys, combined at the
// end across the key splits by their log-sum-exp. The fp32 path serves small,
// launch-latency-bound shapes (one head of 128 rows is 2 MFLOP), so it is
// built for a short critical path rather than for throughput:
//
//   - a work-group (4 waves) owns 4 query rows; each wave takes every 4th block
//     of 8 keys, so the keys of a row are split four ways;
//   - inside a wave, 16 lanes share a row, each holding d/16 consecutive dims
//     of q and of its accumulator (d = 32, 64, 96, 128 or 256); a score is a
//     d/16-FMA partial dot product and a 16-lane sum over DPP (quad permutes,
//     then half-row and row mirrors);
//   - K and V rows are read straight from global memory as float4s, or
//     float2s where d/16 is not a multiple of 4 (the four
//     rows of a wave read the same addresses, which the cache merges), so no
//     LDS staging and no barrier sits on the path;
//   - probabilities use exp2 of scores pre-multiplied by scale*log2(e);
//   - the four waves' (max, sum, accumulator) states are merged through LDS.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRowsPerWG = 4;  // query rows per work-group (one per 16 lanes)
constexpr int kSplit = 4;      // waves = key splits
constexpr int kKB = 8;         // keys per block

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
  return x;
}

// DP consecutive floats: float4 accesses when DP is a multiple of 4, else
// float2 (d = 32, 96); the row offsets keep them 16- or 8-byte aligned.
template <int DP>
__device__ __forceinline__ void load_dp(const float* src, float* dst) {
  if constexpr (DP % 4 == 0) {
#pragma unroll
    for (int e = 0; e < DP; e += 4) {
      const float4 x = *(const float4*)(src + e);
      dst[e] = x.x; dst[e + 1] = x.y; dst[e + 2] = x.z; dst[e + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < DP; e += 2) {
      const float2 x = *(const float2*)(src + e);
      dst[e] = x.x; dst[e + 1] = x.y;
    }
  }
}
template <int DP>
__device__ __forceinline__ void store_dp(float* dst, const float* src, float f) {
  if constexpr (DP % 4 == 0) {
#pragma unroll
    for (int e = 0; e < DP; e += 4) *(float4*)(dst + e) = make_float4(src[e] * f, src[e + 1] * f, src[e + 2] * f, src[e + 3] * f);
  } else {
#pragma unroll
    for (int e = 0; e < DP; e += 2) *(float2*)(dst + e) = make_float2(src[e] * f, src[e + 1] * f);
  }
}

template <int D>
__global__ void __launch_bounds__(256) prefill_f32_kernel(PrefillParams p) {
  constexpr int DP = D / 16;  // dims per lane
  __shared__ __attribute__((aligned(16))) float sAcc[kSplit][kRowsPerWG][D];
  __shared__ float sM[kSplit][kRowsPerWG], sL[kSplit][kRowsPerWG];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rr = lane >> 4, t = lane & 15;
  const int r0 = blockIdx.x * kRowsPerWG;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq, Skv = p.Skv, off = Skv - Sq;
  const bool causal = p.causal != 0;
  const int row = r0 + rr;
  const bool valid = row < Sq;
  const float cs = p.neg ? -p.c : p.c;  // scale * log2(e)

  float q[DP], acc[DP];
  {
    const float* qrow = (const float*)p.q + (((size_t)b * p.Hq + h) * Sq + (valid ? row : 0)) * D + t * DP;
    load_dp<DP>(qrow, q);
    if (!valid)
#pragma unroll
      for (int e = 0; e < DP; ++e) q[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DP; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  // keys any row of this work-group can see; the last key this row can see
  const int last_row = min(Sq, r0 + kRowsPerWG) - 1;
  const int kend = causal ? min(Skv, last_row + off + 1) : Skv;
  const int lim = causal ? min(row + off, Skv - 1) : Skv - 1;
  const int nblk = (kend + kKB - 1) / kKB;
  const float* kbh = (const float*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D + t * DP;
  const float* vbh = (const float*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D + t * DP;

  for (int blk = w; blk < nblk; blk += kSplit) {
    const int k0 = blk * kKB;
    float kv[kKB][DP], vv[kKB][DP];
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      const size_t key = (size_t)min(k0 + j, Skv - 1);  // rows past Skv are masked below
      load_dp<DP>(kbh + key * D, kv[j]);
      load_dp<DP>(vbh + key * D, vv[j]);
    }
    float s[kKB];
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      float sp = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) sp = fmaf(q[e], kv[j][e], sp);
      sp = row16_sum(sp) * cs;
      s[j] = (k0 + j <= lim) ? sp : -INFINITY;
      bm = fmaxf(bm, s[j]);
    }
    const float mn = fmaxf(m, bm);
    if (mn == -INFINITY) continue;  // nothing of this block is visible to this row yet
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      const float pj = __builtin_amdgcn_exp2f(s[j] - mn);  // exp2(-inf) = 0 for masked keys
      l += pj;
#pragma unroll
      for (int e = 0; e < DP; ++e) acc[e] = fmaf(pj, vv[j][e], acc[e]);
    }
  }

  // merge the four key splits: o = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w
#pragma unroll
  for (int e = 0; e < DP; ++e) sAcc[w][rr][t * DP + e] = acc[e];
  if (t == 0) {
    sM[w][rr] = m;
    sL[w][rr] = l;
  }
  __syncthreads();
  if (w != 0 || !valid) return;
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kSplit; ++u) M = fmaxf(M, sM[u][rr]);
  float L = 0.f, o[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) o[e] = 0.f;
#pragma unroll
  for (int u = 0; u < kSplit; ++u) {
    const float mu = sM[u][rr];
    const float f = (mu == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mu - M);
    L = fmaf(f, sL[u][rr], L);
#pragma unroll
    for (int e = 0; e < DP; ++e) o[e] = fmaf(f, sAcc[u][rr][t * DP + e], o[e]);
  }
  const float inv = 1.0f / L;
  float* orow = (float*)p.o + (((size_t)b * p.Hq + h) * Sq + row) * D + t * DP;
  store_dp<DP>(orow, o, inv);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream) {
  dim3 grid((p.Sq + kRowsPerWG - 1) / kRowsPerWG, p.Hq, p.B), block(256);
  if (d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, stream, p);
  else if (d == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, stream, p);
  else if (d == 32)
    hipLaunchKernelGGL(prefill_f32_kernel<32>, grid, block, 0, stream, p);
  else if (d == 96)
    hipLaunchKernelGGL(prefill_f32_kernel<96>, grid, block, 0, stream, p);
  else if (d == 256)
    hipLaunchKernelGGL(prefill_f32_kernel<256>, grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
