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

// ---------------------------------------------------------------------------
// Large shapes: the same attention on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32, full fp32 products and sums), for d = 32, 64, 96
// and 128. One work-group of 4 waves per (128-row query tile, head, batch);
// each wave owns 32 query rows; K and V blocks of 32 keys come into LDS by
// direct-to-LDS loads, double-buffered, one barrier per block. Every head
// dim fits in 256 registers with 64 KB of LDS or less, so two work-groups
// share a CU and one's MFMAs run while the other's softmax and loads do.
// Operand reads are a per-lane base plus a constant and are issued a few
// MFMAs ahead of their use.
//
// The contraction order is permuted so that every operand comes whole from
// 16-byte pieces: in k-step (m, e) lane half hl (lanes 32 hl .. 32 hl + 31)
// contracts index 8m + 4hl + e (e = 0..3). For S^T = K . Q^T the index is a
// dim: a lane reads dims 8m + 4hl .. +3 of its key with one 16-byte LDS read
// and holds those of its query in registers. For O^T = V^T . P^T the index is
// a key: the score accumulator of a lane already holds keys 8m + 4hl + e in
// its registers 4m + e (the 32x32 output layout), so the probabilities are
// the B operand in place, in fp32; V^T comes as four 4-byte LDS reads.
constexpr int kKNf = 32;        // keys per block
constexpr float kTauF = 8.0f;   // lazy rescale threshold (log2 units)
constexpr int kXcdsF = 8;
constexpr int kCusF = 256;     // compute units of an MI355X
constexpr int kRsrcW3F = 0x00020000;

template <int N>
struct StageF {
  static constexpr int value = N;
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_f32_mfma_kernel(PrefillParams p) {
  constexpr int CH = D / 4;              // 16-byte chunks per fp32 row
  constexpr int STAGE = kKNf * D;        // floats per K or V block
  constexpr int NI = kKNf * CH / 64 / 4; // direct-to-LDS loads per wave per block
  constexpr int DB = D / 32;             // 32-dim blocks of O^T
  constexpr int KM = D / 8;              // groups of 4 k-steps of S^T
  __shared__ __attribute__((aligned(1024))) float sK0[STAGE];
  __shared__ __attribute__((aligned(1024))) float sV0[STAGE];
  __shared__ __attribute__((aligned(1024))) float sK1[STAGE];
  __shared__ __attribute__((aligned(1024))) float sV1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  int t, h, b;
  const int W = p.nT * p.Hq * p.B;
  if (p.causal && W <= 2 * kCusF) {
    // One round, two work-groups per CU: the dispatcher gives the first kCusF
    // work-groups one CU each and the rest the second slot of the same CUs in
    // the same order. Items ranked by cost (tile from the most keys down, then
    // head and sequence): the first pass takes them from the top, the second
    // from the bottom, so each CU holds a costly and a cheap tile instead of
    // two alike.
    const int L = blockIdx.x, F = min(W, kCusF), HB = p.Hq * p.B;
    const int r = L < F ? L : W - 1 - (L - F);
    t = p.nT - 1 - r / HB;
    h = (r % HB) % p.Hq;
    b = (r % HB) / p.Hq;
  } else {
    // Work item I: query tile fastest (most keys first), then head, then
    // sequence; each XCD takes a contiguous range of items.
    const int L = blockIdx.x;
    const int xcd = L % kXcdsF, idx = L / kXcdsF;
    const int qq = W / kXcdsF, rr = W % kXcdsF;
    const int I = (xcd < rr) ? xcd * (qq + 1) + idx : rr * (qq + 1) + (xcd - rr) * qq + idx;
    t = p.nT - 1 - I % p.nT;
    h = (I / p.nT) % p.Hq;
    b = I / (p.nT * p.Hq);
  }
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq, Skv = p.Skv, off = Skv - Sq;
  const bool causal = p.causal != 0;
  const float c = p.c;
  const int q_last = min(t * 128 + 128, Sq) - 1;
  const int kend = causal ? min(Skv, q_last + off + 1) : Skv;
  const int nblk = (kend + kKNf - 1) / kKNf;

  const float* kbh = (const float*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const float* vbh = (const float*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const float* qbh = (const float*)p.q + ((size_t)b * p.Hq + h) * (size_t)Sq * D;

  // LDS chunk P of a block holds logical chunk (P % CH) ^ (row % 8) of row
  // P / CH (CH is a multiple of 8): the 16-byte K reads of 8 consecutive rows
  // at one chunk land in 8 distinct bank groups.
  uint32_t off_[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int P = 64 * (wave * NI + ii) + lane;
    const int row = P / CH, pc = P % CH;
    off_[ii] = (uint32_t)(row * D * 4 + ((pc ^ (row & 7)) << 4));
  }
  auto dma = [&](const float* src, float* stage, int j) __attribute__((always_inline)) {
    const int kv0 = j * kKNf;
    const int rows = min(kKNf, Skv - kv0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)kv0 * D), (short)0, rows * D * 4, kRsrcW3F);
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + 64 * (wave * NI + ii) * 4), 16,
                                               (int)off_[ii], 0, 0, 0);
  };

  // Q^T operand: lane (query ln, half hl) holds dims 8m + 4hl .. +3 of its row;
  // a negative scale flips the sign here (exact), so c >= 0.
  const int qrow = t * 128 + wave * 32 + ln;
  const float qs = p.neg ? -1.f : 1.f;
  float4 qreg[KM];
#pragma unroll
  for (int m = 0; m < KM; ++m) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (qrow < Sq) x = *(const float4*)(qbh + (size_t)qrow * D + 8 * m + 4 * hl);
    qreg[m] = make_float4(x.x * qs, x.y * qs, x.z * qs, x.w * qs);
  }

  f32x16 O[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) O[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int q0 = t * 128 + wave * 32;

  // LDS read offsets, per lane, so that every operand read below is a base
  // register plus a constant:
  //   K (S^T, group m = 4a + r of 4 k-steps): row ln, 16-byte chunk
  //   (2m + hl) ^ (ln % 8) = 8a + ((2r + hl) ^ (ln % 8)) -> kofs[r] + 128 a;
  //   V (O^T, k-step (m, e), dim block db): row 8m + 4hl + e, dim 32 db + ln,
  //   chunk (8 db + ln / 4) ^ (4hl + e) -> vofs[e] + 4 ((8m + e) D + 32 db).
  int kofs[4], vofs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    kofs[r] = ln * (D * 4) + (((2 * r + hl) ^ (ln & 7)) << 4);
    vofs[r] = 4 * (4 * hl * D + (((ln >> 2) ^ (4 * hl + r)) << 2) + (ln & 3));
  }

  if (nblk > 0) {
    dma(kbh, sK0, 0);
    dma(vbh, sV0, 0);
  }
  // The loop runs two blocks per iteration with the stages named at compile
  // time, so the compiler tells a block's operand reads from the loads still
  // in flight into the other stage and does not make the reads wait for them.
  auto step = [&](auto stage, int j) __attribute__((always_inline)) {
    constexpr bool odd = decltype(stage)::value != 0;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block j
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads of the other stage are done
    __syncthreads();
    if (j + 1 < nblk) {
      dma(kbh, odd ? sK0 : sK1, j + 1);
      dma(vbh, odd ? sV0 : sV1, j + 1);
    }
    const int kv0 = j * kKNf;
    if (causal && kv0 > q0 + 31 + off) return;  // above every row of this wave
    const char* kb = (const char*)(odd ? sK1 : sK0);
    const float* vb = odd ? sV1 : sV0;

    // S^T (32 keys x 32 queries): lane (query ln, half hl) register r holds
    // key kv0 + 8 (r / 4) + 4 hl + r % 4
    // two accumulation chains (even and odd m), added at the end: half the
    // sequential rounding of one chain over all d products
    f32x16 S = f32x16{}, S2 = f32x16{};
    {
      // K operands read kPFK groups ahead of their MFMAs
      constexpr int kPFK = KM < 3 ? KM : 3;
      auto kread = [&](int m) __attribute__((always_inline)) {
        return *(const float4*)(kb + kofs[m & 3] + 128 * (m >> 2));
      };
      float4 kbuf[kPFK];
#pragma unroll
      for (int i = 0; i < kPFK; ++i) kbuf[i] = kread(i);
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const float4 kx = kbuf[m % kPFK];
        if (m + kPFK < KM) kbuf[m % kPFK] = kread(m + kPFK);
        f32x16& A = (m & 1) ? S2 : S;
        A = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.x, qreg[m].x, A, 0, 0, 0);
        A = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.y, qreg[m].y, A, 0, 0, 0);
        A = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.z, qreg[m].z, A, 0, 0, 0);
        A = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.w, qreg[m].w, A, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] += S2[r];
    const bool full = kv0 + kKNf <= Skv && (!causal || kv0 + kKNf - 1 <= q0 + off);
    if (!full) {
      const int kb0 = kv0 + 4 * hl;
      int lim = Skv - 1 - kb0;
      if (causal) lim = min(lim, qrow + off - kb0);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) S[r] = -INFINITY;
    }
    float mx = S[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
    float alpha = 1.f;
    if (cand > m_run + kTauF) {
      alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - cand);
      m_run = cand;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c, -mu));
      ls += S[r];
    }
    l_run = alpha * l_run + ls;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    // O^T += V^T . P^T: k-step (m, e) contracts key 8m + 4hl + e, whose
    // probability is this lane's register 4m + e. MFMA n of the stream is
    // (m, e, db) = (n / (4 DB), (n / DB) % 4, n % DB); its V^T operand is read
    // kPFV MFMAs ahead.
    {
      constexpr int kNV = 16 * DB;
      constexpr int kPFV = 8;
      const char* vbb = (const char*)vb;
      auto vread = [&](int n) __attribute__((always_inline)) {
        const int m = n / (4 * DB), e = (n / DB) & 3, db = n % DB;
        return *(const float*)(vbb + vofs[e] + 4 * ((8 * m + e) * D + 32 * db));
      };
      float vbuf[kPFV];
#pragma unroll
      for (int i = 0; i < kPFV; ++i) vbuf[i] = vread(i);
#pragma unroll
      for (int n = 0; n < kNV; ++n) {
        const float vx = vbuf[n % kPFV];
        if (n + kPFV < kNV) vbuf[n % kPFV] = vread(n + kPFV);
        const int m = n / (4 * DB), e = (n / DB) & 3, db = n % DB;
        O[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vx, S[4 * m + e], O[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int j = 0; j < nblk; j += 2) {
    step(StageF<0>{}, j);
    if (j + 1 < nblk) step(StageF<1>{}, j + 1);
  }

  // normalise and store: lane (query ln, half hl) register r of O[db] holds
  // dim 32 db + 8 (r / 4) + 4 hl + r % 4
  float lt;
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float inv = 1.0f / lt;
  if (qrow < Sq) {
    float* dst = (float*)p.o + (((size_t)b * p.Hq + h) * Sq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        *(float4*)(dst + 32 * db + 8 * a4 + 4 * hl) =
            make_float4(O[db][4 * a4] * inv, O[db][4 * a4 + 1] * inv, O[db][4 * a4 + 2] * inv,
                        O[db][4 * a4 + 3] * inv);
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream) {
  // Grids of at least 64 query tiles of 128 rows (over heads and batch) take
  // the matrix-core kernel (d <= 128); smaller ones, bound by launch latency
  // or by too few work-groups for the CUs, take the vector kernel, whose
  // work-groups own 4 rows each (measured: the vector kernel is faster up to
  // 32 tiles, the two are even near 48, the matrix cores faster from 64).
  if (d <= 128 && (long)p.nT * p.Hq * p.B >= 64) {
    const dim3 grid(p.nT * p.Hq * p.B), block(256);
    if (d == 128)
      return launch_kernel(prefill_f32_mfma_kernel<128>, grid, block, stream, p);
    else if (d == 64)
      return launch_kernel(prefill_f32_mfma_kernel<64>, grid, block, stream, p);
    else if (d == 96)
      return launch_kernel(prefill_f32_mfma_kernel<96>, grid, block, stream, p);
    else if (d == 32)
      return launch_kernel(prefill_f32_mfma_kernel<32>, grid, block, stream, p);
    else
      return hipErrorInvalidValue;
  }
  dim3 grid((p.Sq + kRowsPerWG - 1) / kRowsPerWG, p.Hq, p.B), block(256);
  if (d == 128)
    return launch_kernel(prefill_f32_kernel<128>, grid, block, stream, p);
  else if (d == 64)
    return launch_kernel(prefill_f32_kernel<64>, grid, block, stream, p);
  else if (d == 32)
    return launch_kernel(prefill_f32_kernel<32>, grid, block, stream, p);
  else if (d == 96)
    return launch_kernel(prefill_f32_kernel<96>, grid, block, stream, p);
  else if (d == 256)
    return launch_kernel(prefill_f32_kernel<256>, grid, block, stream, p);
  else
    return hipErrorInvalidValue;
}

}  // namespace fa
