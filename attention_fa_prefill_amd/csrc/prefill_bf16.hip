// prefill_bf16.hip - fused causal / non-causal MQA/GQA attention, bf16 in/out,
// on gfx950 MFMA.
//
// What it computes is the tiled attention of the "Real-time inference
// optimisation" page (section "Flash Attention optimisation"): per query row a
// running max m, a running sum l and an accumulator rescaled by exp(m_old -
// m_new) while K/V tiles stream past, normalised by l at the end; plus the
// causal mask and MQA/GQA head sharing listed on the FlashRT-HF-kernels page
// (section "attention optimisation"). The score matrix never leaves registers.
//
// Work decomposition (one work-group = 512 threads = two groups of 4 waves;
// each wave owns 32 query rows, so a group owns a 128-row query tile):
//   - work-group p of head (b, h) takes query tiles t0 = p and t1 = nT-1-p. With
//     a causal mask tile t needs ~t+1 KV blocks, so t0 + t1 always needs about
//     the same work. Group B runs the first half of t1's KV range; group A runs
//     all of t0 and then the rest of t1's range; the two partial states of t1
//     (m, l, O) are merged through LDS. Every work-group gets the same work.
//   - K/V blocks of 64 keys go HBM -> LDS with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4), double-buffered per group; the next block is in
//     flight while the current one is consumed.
//
// Per wave and per 64-key block (two 32-key sub-tiles):
//   S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T held
//   in VGPRs), so each lane holds 16 scores of one query; the row max needs only
//   an in-lane max and one v_permlane32_swap with the other half-wave.
//   P = exp2(S*c - m) with c = scale*log2(e); the running max is raised lazily
//   (only when it grows by more than kTau, in log2 units), which changes no
//   result in exact arithmetic and skips most accumulator rescales.
//   O^T += V^T . P^T on the same MFMA: A = V^T read with ds_read_b64_tr_b16
//   from the row-major V tile in LDS, B = P^T straight from the score registers
//   (the contraction order over keys is permuted to match their lane layout).
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 128;     // query rows per wave group
constexpr int kBN = 64;      // keys per KV block
constexpr float kTau = 8.0f; // lazy rescale threshold (log2 units)

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;               // 16-byte chunks per K/V row
  static constexpr int ELEMS = kBN * D;          // bf16 elements per K or V block
  static constexpr int NI = kBN * CH / 64 / 4;   // direct-to-LDS loads per wave per block
  static constexpr int KS = D / 16;              // k-steps of S^T = K . Q^T
  static constexpr int DB = D / 32;              // 32-row d blocks of O^T
  static constexpr int XO = 64 * DB * 16;        // floats of one wave's O^T in the exchange
};

// LDS swizzles (16-byte chunk index XOR a function of the row).
// K rows are read 16 bytes per lane for 16 consecutive rows at one chunk:
// XOR with row mod CH spreads them over all banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (Cfg<D>::CH - 1); }
// V is read by transpose reads: each 16-lane group touches 4 consecutive rows x
// 32 bytes. XOR with 2*(row%4) (D=64) / 4*(row%4) (D=128) places those 4 rows
// in different bank windows and keeps each 32-byte pair of chunks together.
template <int D>
__device__ __forceinline__ int swz_v(int row) { return (D == 128 ? 4 : 2) * (row & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Issue one 64-key K or V block of one group: HBM -> LDS, 16 bytes per lane.
// LDS chunk P of the block holds logical chunk (P % CH) ^ swz(row) of row
// P / CH; rows past Skv are clamped to Skv-1 (finite data, masked out later).
template <int D, bool IS_V>
__device__ __forceinline__ void dma_block(const __bf16* __restrict__ src_bh, __bf16* lds_block, int kv0, int Skv,
                                          int wg, int lane) {
  using C = Cfg<D>;
#pragma unroll
  for (int ii = 0; ii < C::NI; ++ii) {
    const int P = 64 * (wg * C::NI + ii) + lane;
    const int row = P / C::CH, pc = P % C::CH;
    const int lc = pc ^ (IS_V ? swz_v<D>(row) : swz_k<D>(row));
    const int grow = min(kv0 + row, Skv - 1);
    const __bf16* src = src_bh + (size_t)grow * D + lc * 8;
    __bf16* dst = lds_block + 64 * (wg * C::NI + ii) * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)dst, 16, 0, 0);
  }
}

template <int D>
__global__ void __launch_bounds__(512) prefill_bf16_kernel(PrefillParams p) {
  using C = Cfg<D>;
  // Two stages x {K, V}, each holding both groups' blocks. Separate arrays let
  // the compiler see that the block being loaded never aliases the block being
  // read, so no wait is inserted between them.
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[2 * C::ELEMS];

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: keep it (and everything derived
  // from it) in scalar registers so that per-wave decisions are scalar branches.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0 = group A, 1 = group B
  const int wg = wave & 3;    // wave within group
  const int hl = lane >> 5;   // half-wave
  const int ln = lane & 31;
  const int pidx = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq, Skv = p.Skv;
  const int off = Skv - Sq;
  const bool causal = p.causal != 0;
  const float c = p.c;

  auto nblocks = [&](int t) __attribute__((always_inline)) {
    const int end = causal ? min(Skv, (t + 1) * kBM + off) : Skv;
    return (end + kBN - 1) / kBN;
  };
  const int t0 = pidx, t1 = p.nT - 1 - pidx;
  const int n1 = nblocks(t1);
  const int nA0 = (t0 == t1) ? 0 : nblocks(t0);
  const int jB = min(n1, (nA0 + n1 + 1) / 2);  // group B: t1 blocks [0, jB)
  const int cntA = nA0 + (n1 - jB), cntB = jB;
  const bool split = jB < n1;                  // group A holds a partial of t1
  const int cnt = grp ? cntB : cntA;
  const int maxcnt = max(cntA, cntB);
  auto kv_of = [&](int i) __attribute__((always_inline)) { return grp ? i : (i < nA0 ? i : jB + (i - nA0)); };

  const __bf16* kbh = (const __bf16*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* vbh = (const __bf16*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;

  // Per-lane byte offsets (inside a 64-key block) of this lane's direct-to-LDS
  // loads: LDS chunk P of the block holds logical chunk (P % CH) ^ swz(row) of
  // row P / CH. Loop-invariant, so a full block costs one scalar base per load.
  uint32_t koff[C::NI], voff[C::NI];
#pragma unroll
  for (int ii = 0; ii < C::NI; ++ii) {
    const int P = 64 * (wg * C::NI + ii) + lane;
    const int row = P / C::CH, pc = P % C::CH;
    koff[ii] = (uint32_t)(row * D + ((pc ^ swz_k<D>(row)) << 3)) * 2u;
    voff[ii] = (uint32_t)(row * D + ((pc ^ swz_v<D>(row)) << 3)) * 2u;
  }
  auto dma = [&](__bf16* sK, __bf16* sV, int j) __attribute__((always_inline)) {
    const int kv0 = j * kBN;
    __bf16* kd = sK + grp * C::ELEMS;
    __bf16* vd = sV + grp * C::ELEMS;
    if (kv0 + kBN <= Skv) {
      const char* kb = (const char*)(kbh + (size_t)kv0 * D);
      const char* vb = (const char*)(vbh + (size_t)kv0 * D);
#pragma unroll
      for (int ii = 0; ii < C::NI; ++ii) {
        __bf16* dst = 64 * (wg * C::NI + ii) * 8 + kd;
        __builtin_amdgcn_global_load_lds((const void*)(kb + koff[ii]), (lds_void_t*)dst, 16, 0, 0);
      }
#pragma unroll
      for (int ii = 0; ii < C::NI; ++ii) {
        __bf16* dst = 64 * (wg * C::NI + ii) * 8 + vd;
        __builtin_amdgcn_global_load_lds((const void*)(vb + voff[ii]), (lds_void_t*)dst, 16, 0, 0);
      }
    } else {
      dma_block<D, false>(kbh, kd, kv0, Skv, wg, lane);
      dma_block<D, true>(vbh, vd, kv0, Skv, wg, lane);
    }
  };

  f32x16 O[C::DB];
  bf16x8 qreg[C::KS];
  float m_run = -INFINITY, l_run = 0.f;

  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[db][r] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // Q^T operand: lane holds Q[row ln][16 ks + 8 hl .. +8] for every k-step.
  auto load_q = [&](int t) __attribute__((always_inline)) {
    const int row = t * kBM + wg * 32 + ln;
    const uint32_t flip = p.neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < Sq) {
        const uint4* src = (const uint4*)((const __bf16*)p.q + (((size_t)b * p.Hq + h) * Sq + row) * D + 16 * ks + 8 * hl);
        x = *src;
      }
      x.x ^= flip; x.y ^= flip; x.z ^= flip; x.w ^= flip;
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  };

  auto store_tile = [&](int t) __attribute__((always_inline)) {
    const float lt = pair_sum(l_run);
    const float inv = 1.0f / lt;
    const int row = t * kBM + wg * 32 + ln;
    if (row < Sq) {
      __bf16* dst = (__bf16*)p.o + (((size_t)b * p.Hq + h) * Sq + row) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          uint2 w;
          w.x = pack_bf16x2(O[db][4 * rg + 0] * inv, O[db][4 * rg + 1] * inv);
          w.y = pack_bf16x2(O[db][4 * rg + 2] * inv, O[db][4 * rg + 3] * inv);
          *(uint2*)(dst + 32 * db + 8 * rg + 4 * hl) = w;
        }
    }
  };

  const int kr0 = ln * (D * 2), kr1 = (32 + ln) * (D * 2);
  const int sw0 = swz_k<D>(ln), sw1 = swz_k<D>(32 + ln);
  auto kread = [&](const char* kbase, int kr, int sw, int ks) __attribute__((always_inline)) {
    return *(const bf16x8*)(kbase + kr + (((2 * ks + hl) ^ sw) << 4));
  };
  // V^T operand rows/columns (transpose reads): see the header comment.
  const int gg = lane >> 4, jj = lane & 15, dh = gg & 1;
  auto vread = [&](const char* vbase, int sub, int s, int db) __attribute__((always_inline)) {
    const int row1 = 32 * sub + 16 * s + 4 * hl + (jj >> 2);
    const int row2 = row1 + 8;
    const int colb = (32 * db + 16 * dh + 4 * (jj & 3)) * 2;
    const char* a1 = vbase + row1 * (D * 2) + (((colb >> 4) ^ swz_v<D>(row1)) << 4) + (colb & 15);
    const char* a2 = vbase + row2 * (D * 2) + (((colb >> 4) ^ swz_v<D>(row2)) << 4) + (colb & 15);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Online-softmax update from the tile max; returns the rescale factor.
  auto update_max = [&](float mx) __attribute__((always_inline)) {
    mx = pair_max(mx);
    const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
    float alpha = 1.f;
    if (cand > m_run + kTau) {
      alpha = fast_exp2(m_run - cand);
      m_run = cand;
    }
    return alpha;
  };
  auto rescale = [&](float alpha, float lsum) __attribute__((always_inline)) {
    l_run = alpha * l_run + lsum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
  };
  // exp2, row-sum and bf16 packing of one 32-key sub-tile. Masked scores are
  // -inf and come out as exactly 0 (c > 0 and mu finite).
  auto probs = [&](const f32x16& Ssub, float mu, bf16x8* P2, float& la, float& lb) __attribute__((always_inline)) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(Ssub[r], c, -mu));
#pragma unroll
    for (int r = 0; r < 16; r += 2) { la += e[r]; lb += e[r + 1]; }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 w;
      w.x = pack_bf16x2(e[8 * s + 0], e[8 * s + 1]);
      w.y = pack_bf16x2(e[8 * s + 2], e[8 * s + 3]);
      w.z = pack_bf16x2(e[8 * s + 4], e[8 * s + 5]);
      w.w = pack_bf16x2(e[8 * s + 6], e[8 * s + 7]);
      P2[s] = __builtin_bit_cast(bf16x8, w);
    }
  };
  auto pv = [&](const char* vbase, int sub, const bf16x8* P2) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a = vread(vbase, sub, s, 0);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        bf16x8 an = a;
        if (db + 1 < C::DB) an = vread(vbase, sub, s, db + 1);
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P2[s], O[db], 0, 0, 0);
        a = an;
      }
    }
  };

  // One 64-key block for this wave's 32 rows. Blocks that some row sees only
  // partly (causal diagonal, end of the keys) get their invisible scores set to
  // -inf behind a wave-uniform branch; a block no row of the wave sees is skipped.
  auto block = [&](const __bf16* sK, const __bf16* sV, int q0, int kv0) __attribute__((always_inline)) {
    if (kv0 >= Skv || (causal && kv0 > q0 + 31 + off)) return;
    const char* kbase = (const char*)(sK + grp * C::ELEMS);
    const char* vbase = (const char*)(sV + grp * C::ELEMS);
    f32x16 S0 = f32x16{}, S1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 a0 = kread(kbase, kr0, sw0, ks);
      const bf16x8 a1 = kread(kbase, kr1, sw1, ks);
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], S1, 0, 0, 0);
    }
    const bool full = kv0 + kBN <= Skv && (!causal || kv0 + kBN - 1 <= q0 + off);
    if (!full) {
      // key of register r of sub-tile u is kb + 8*(r/4) + (r%4), kb = kv0 + 32u + 4hl;
      // visible iff < Skv and (non-causal or) <= query row + off
      const int kb = kv0 + 4 * hl;
      int lim = Skv - 1 - kb;
      if (causal) lim = min(lim, q0 + ln + off - kb);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ko = 8 * (r >> 2) + (r & 3);
        if (ko > lim) S0[r] = -INFINITY;
        if (ko + 32 > lim) S1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[r], S1[r]));
    const float alpha = update_max(mx);
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 P0[2], P1[2];
    float la = 0.f, lb = 0.f;
    probs(S0, mu, P0, la, lb);
    probs(S1, mu, P1, la, lb);
    rescale(alpha, la + lb);
    pv(vbase, 0, P0);
    pv(vbase, 1, P1);
  };

  // One iteration: barrier, prefetch the next block into the other stage,
  // consume this block. (sKc, sVc) is this iteration's stage.
  auto body = [&](int i, int t, __bf16* sKc, __bf16* sVc, __bf16* sKn, __bf16* sVn) __attribute__((always_inline)) {
    __syncthreads();
    if (i + 1 < cnt) dma(sKn, sVn, kv_of(i + 1));
    block(sKc, sVc, t * kBM + wg * 32, kv_of(i) * kBN);
  };
  // Iterations [i0, i1) of this group, all on tile t; the stage is the
  // iteration's parity (the loop walks aligned pairs and skips iterations
  // outside the range, so each stage's code appears once).
  auto run = [&](int i0, int i1, int t) __attribute__((always_inline)) {
    for (int i = i0 & ~1; i < i1; i += 2) {
      if (i >= i0) body(i, t, sK0, sV0, sK1, sV1);
      if (i + 1 < i1) body(i + 1, t, sK1, sV1, sK0, sV0);
    }
  };

  // ---- main loops: both groups execute exactly maxcnt barriers.
  // Group A: phase 0 = all of t0, phase 1 = the tail of t1's KV range.
  // Group B: phase 0 = the head of t1's KV range.
  if (cnt > 0) dma(sK0, sV0, kv_of(0));
  for (int phase = 0; phase < 2; ++phase) {
    int i0, i1, t;
    if (grp == 0) {
      i0 = phase ? nA0 : 0;
      i1 = phase ? cntA : nA0;
      t = phase ? t1 : t0;
    } else {
      i0 = 0;
      i1 = phase ? 0 : cntB;
      t = t1;
    }
    if (i0 >= i1) continue;
    reset_state();
    load_q(t);
    run(i0, i1, t);
    if (grp == 0 && phase == 0) store_tile(t0);
  }
  for (int i = cnt; i < maxcnt; ++i) __syncthreads();

  // ---- epilogue: group A hands its partial of t1 to group B through LDS.
  __syncthreads();
  float* xo = (float*)((wg < 2 ? (char*)sK0 : (char*)sV0)) + (wg & 1) * C::XO;
  float* xml = (float*)sK1 + wg * 128;
  if (grp == 0 && split) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = O[db][r];
    xml[lane * 2 + 0] = m_run;
    xml[lane * 2 + 1] = l_run;
  }
  __syncthreads();
  if (grp == 1) {
    if (split) {
      const float mA = xml[lane * 2 + 0], lA = xml[lane * 2 + 1];
      const float m = fmaxf(m_run, mA);
      const float aB = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m);
      const float aA = (mA == -INFINITY) ? 0.f : fast_exp2(mA - m);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] = O[db][r] * aB + xo[(db * 16 + r) * 64 + lane] * aA;
      l_run = l_run * aB + lA * aA;
      m_run = m;
    }
    store_tile(t1);
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
  dim3 grid(p.nP, p.Hq, p.B), block(512);
  if (d == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
