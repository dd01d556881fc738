// decode.hip - single-token decode over a contiguous or paged bf16 KV cache
// (split-KV), and the log-sum-exp merge of the splits.
//
// Decode reads every cached K and V byte once and does ~Hq/Hkv FLOP per byte,
// so it is bound by HBM bandwidth (the generation phase is memory-bound: the
// FasterTransformer source review, sections 1.1 and 3.1). The paged layout is
// the one of the "Real-time inference optimisation" page's paged sketch (pages
// of 16 tokens); where that sketch adds the per-page outputs, which is wrong,
// the splits here are combined by log-sum-exp.
//
// Split kernel: one work-group (4 waves) per (sequence b, kv head g, group of
// up to 16 query heads sharing g, split s of tps tokens). Waves take 32-token
// steps round-robin. Per step:
//   - K rows go HBM -> VGPRs directly in the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (16 tokens x 32 dims per MFMA);
//   - S^T = K . Q^T for all query heads of the group at once (Q^T lives in
//     VGPRs; unused head columns are zero), so the FLOPs ride on MFMA and the
//     vector ALU only runs the softmax;
//   - V rows go HBM -> VGPRs -> the wave's own LDS slot, then come back through
//     ds_read_b64_tr_b16 as the A operand of O^T += V^T . P^T;
//   - online softmax per head with a lazily raised running max.
// The next step's K and V loads are issued before the current step is used.
// Tokens past the sequence length get score -inf and a zero V row (never a NaN
// times zero); block-table entries past the last page are never read.
// At the end the 4 waves' states are merged in LDS and the split writes its
// normalised output and natural-log log-sum-exp to the workspace.
//
// Paged and contiguous caches run the same instructions in the same order and
// differ only in the row address, so their results are bitwise equal.
//
// Merge kernel: per (row, 32 output dims), M = max lse_s, w_s = exp(lse_s - M),
// o = sum_s w_s o_s / sum_s w_s, lse = M + log(sum_s w_s); empty splits skipped.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kStep = 32;      // tokens per wave step
constexpr float kTau = 8.0f;   // lazy rescale threshold (log2 units)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// V staging swizzle: 16-byte chunk XOR 2*(row % 8) (D=128) / 2*(row % 4) (D=64),
// so the 4-row x 32-byte footprint of each transpose read hits distinct banks.
template <int D>
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & (D == 128 ? 7 : 3)); }

template <int D>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeParams p) {
  constexpr int KS = D / 32;         // k-steps of S^T = K . Q^T (16x16x32)
  constexpr int DB = D / 16;         // 16-dim blocks of O^T
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int VL = kStep * CH / 64;  // V chunk loads per lane per step
  constexpr int MAXP = 64;           // block-table entries cached per split (tps <= 1024)
  __shared__ __attribute__((aligned(16))) __bf16 sV[4][kStep * D];
  __shared__ float sM[4][64], sL[4][64];
  __shared__ int sRow0[MAXP];        // first cache row of each page of this split

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = blockIdx.x;
  const int g = blockIdx.y / p.hchunks, hc = blockIdx.y % p.hchunks;
  const int b = blockIdx.z;
  int len = p.lens[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int tok0 = s * p.tps;
  if (tok0 >= len) return;  // empty split: the merge never reads it
  const int tok1 = min(len, tok0 + p.tps);
  const int nsteps = (tok1 - tok0 + kStep - 1) / kStep;
  const int hq0 = g * p.G + hc * 16;
  const int nh = min(16, p.G - hc * 16);
  const int Hkv = p.Hkv;

  // First cache row of each 16-token page this split touches.
  const int npg = (tok1 - tok0 + 15) / 16;
  for (int i = tid; i < npg; i += 256) {
    const int pg = tok0 / 16 + i;
    sRow0[i] = p.bt ? p.bt[(size_t)b * p.pages_per_seq + pg] * 16 : b * p.max_len + pg * 16;
  }
  __syncthreads();

  const int n = lane & 15, cq = lane >> 4;  // MFMA column (head) and k-group
  // Q^T operand: lane holds q[b, hq0+n, 32 ks + 8 cq .. +8]; zero columns past nh.
  bf16x8 qop[KS];
  {
    const uint32_t flip = p.neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (n < nh) x = *(const uint4*)((const __bf16*)p.q + ((size_t)b * p.Hq + hq0 + n) * D + 32 * ks + 8 * cq);
      x.x ^= flip; x.y ^= flip; x.z ^= flip; x.w ^= flip;
      qop[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const __bf16* kc = (const __bf16*)p.kc;
  const __bf16* vc = (const __bf16*)p.vc;
  auto row_of = [&](int tok) { return (size_t)(sRow0[(tok - tok0) >> 4] + (tok & 15)); };

  // K operand registers for one step: [half][ks], token = tb + 16 half + n.
  bf16x8 kreg[2][KS];
  uint4 vreg[VL];
  auto load_step = [&](int st) {
    const int tb = tok0 + st * kStep;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tok = tb + 16 * half + n;
      const bool ok = tok < tok1;
      const __bf16* src = kc + (row_of(ok ? tok : tb) * Hkv + g) * D + 8 * cq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (ok) x = *(const uint4*)(src + 32 * ks);
        kreg[half][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
#pragma unroll
    for (int ii = 0; ii < VL; ++ii) {
      const int P = 64 * ii + lane;
      const int r = P / CH, ch = P % CH;
      const int tok = tb + r;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tok < tok1) x = *(const uint4*)(vc + (row_of(tok) * Hkv + g) * D + ch * 8);
      vreg[ii] = x;
    }
  };

  f32x4 O[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;
  char* vslot = (char*)sV[w];

  int st = w;
  if (st < nsteps) load_step(st);
  for (; st < nsteps; st += 4) {
    const int tb = tok0 + st * kStep;
    // S^T = K . Q^T for the two 16-token halves
    f32x4 S[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      S[half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        S[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kreg[half][ks], qop[ks], S[half], 0, 0, 0);
    }
    // stage V into this wave's LDS slot (swizzled)
#pragma unroll
    for (int ii = 0; ii < VL; ++ii) {
      const int P = 64 * ii + lane;
      const int r = P / CH, ch = P % CH;
      *(uint4*)(vslot + r * (D * 2) + ((ch ^ swz_v<D>(r)) << 4)) = vreg[ii];
    }
    // prefetch the next step of this wave
    if (st + 4 < nsteps) load_step(st + 4);

    // mask tokens past the end: S^T lane (n, cq) reg r is token tb + 16 half + 4 cq + r
    const bool tail = tb + kStep > tok1;
    if (tail) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tb + 16 * half + 4 * cq + r >= tok1) S[half][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[half][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
    float alpha = 1.f;
    if (cand > m_run + kTau) {
      alpha = fast_exp2(m_run - cand);
      m_run = cand;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    float e[8];
    float lsum = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = fast_exp2(fmaf(S[half][r], c, -mu));
        if (tail && S[half][r] == -INFINITY) x = 0.f;
        e[4 * half + r] = x;
        lsum += x;
      }
    l_run = alpha * l_run + lsum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) O[db] *= alpha;
    }
    uint4 pw;
    pw.x = pack_bf16x2(e[0], e[1]);
    pw.y = pack_bf16x2(e[2], e[3]);
    pw.z = pack_bf16x2(e[4], e[5]);
    pw.w = pack_bf16x2(e[6], e[7]);
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);

    // the slot was written by this wave only: order its writes before the reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T . P^T; contraction index 8 cq + i is token 4 cq + i (i < 4)
    // or 16 + 4 cq + (i - 4) (i >= 4), matching the score registers.
    const int y = lane & 15;
    const int row1 = 4 * cq + (y >> 2), row2 = 16 + 4 * cq + (y >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int colb = (16 * db + 4 * (y & 3)) * 2;
      const char* a1 = vslot + row1 * (D * 2) + (((colb >> 4) ^ swz_v<D>(row1)) << 4) + (colb & 15);
      const char* a2 = vslot + row2 * (D * 2) + (((colb >> 4) ^ swz_v<D>(row2)) << 4) + (colb & 15);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop, O[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the 4 waves: O^T lane (n, cq) reg r is dim 16 db + 4 cq + r of head n.
  __syncthreads();
  float* xo = (float*)sV[w];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) xo[(db * 4 + r) * 64 + lane] = O[db][r];
  sM[w][lane] = m_run;
  sL[w][lane] = l_run;
  __syncthreads();
  if (w != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) M = fmaxf(M, sM[u][lane]);
  float a[4];
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float mu = sM[u][lane];
    a[u] = (mu == -INFINITY) ? 0.f : fast_exp2(mu - M);
    L += a[u] * sL[u][lane];
  }
  // each lane summed only its own tokens: add the 4 k-groups of the head
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
  const float inv = 1.0f / L;
  if (n < nh) {
    const int hq = hq0 + n;
    float* dst = p.ws_o + (((size_t)b * p.Hq + hq) * p.nsplit + s) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float4 v;
      float acc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) x += a[u] * ((const float*)sV[u])[(db * 4 + r) * 64 + lane];
        acc[r] = x * inv;
      }
      v = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *(float4*)(dst + 16 * db + 4 * cq) = v;
    }
    if (cq == 0) p.ws_lse[((size_t)b * p.Hq + hq) * p.nsplit + s] = (M + __log2f(L)) * kLn2;
  }
}

// Merge: grid (R, D/32), 256 threads = 32 dims x 8 split groups.
__global__ void __launch_bounds__(256) merge_kernel(MergeParams p, int D) {
  __shared__ float red[256];
  __shared__ float acc_s[8][32];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int d = blockIdx.y * 32 + (tid & 31);
  const int sg = tid >> 5;
  int nS = p.S;
  if (p.lens) {
    int len = p.lens[r / p.Hq];
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    nS = (len + p.tps - 1) / p.tps;
  }
  const float* lse = p.lse + (size_t)r * p.S;
  float M = -INFINITY;
  for (int s = tid; s < nS; s += 256) M = fmaxf(M, lse[s]);
  red[tid] = M;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  float acc = 0.f, W = 0.f;
  if (M != -INFINITY) {
    for (int s = sg; s < nS; s += 8) {
      const float ls = lse[s];
      if (ls == -INFINITY) continue;
      const float wgt = expf(ls - M);
      W += wgt;
      acc += wgt * p.o_parts[((size_t)r * p.S + s) * D + d];
    }
  }
  acc_s[sg][tid & 31] = acc;
  red[tid] = W;
  __syncthreads();
  if (sg == 0) {
    float a = 0.f, wsum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a += acc_s[u][tid];
      wsum += red[u * 32 + tid];
    }
    const float val = (M == -INFINITY) ? 0.f : a / wsum;
    if (p.out_bf16)
      ((__bf16*)p.o)[(size_t)r * D + d] = (__bf16)val;
    else
      ((float*)p.o)[(size_t)r * D + d] = val;
    if (p.lse_out && blockIdx.y == 0 && tid == 0) p.lse_out[r] = (M == -INFINITY) ? -INFINITY : M + logf(wsum);
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int d, hipStream_t stream) {
  dim3 grid(p.nsplit, p.Hkv * p.hchunks, p.B), block(256);
  if (d == 128)
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeParams m;
  m.o_parts = p.ws_o;
  m.lse = p.ws_lse;
  m.o = p.o;
  m.lse_out = nullptr;
  m.lens = p.lens;
  m.R = p.B * p.Hq;
  m.S = p.nsplit;
  m.Hq = p.Hq;
  m.tps = p.tps;
  m.max_len = p.max_len;
  m.out_bf16 = 1;
  return launch_merge(m, d, stream);
}

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t stream) {
  dim3 grid(p.R, d / 32), block(256);
  hipLaunchKernelGGL(merge_kernel, grid, block, 0, stream, p, d);
  return hipGetLastError();
}

}  // namespace fa
