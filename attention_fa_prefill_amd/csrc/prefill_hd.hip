// bf16 prefill for the head dims the ping-pong kernel does not provide
// (d = 32, 96, 256): causal or non-causal MQA/GQA attention with an online
// softmax, fp32 accumulation, bf16 MFMA for both products.
//
// It computes the tiled attention of the "Real-time inference optimisation"
// page (section "Flash Attention optimisation"): the key/value blocks stream
// through on-chip memory while a running row maximum and row sum rescale the
// output accumulator, normalised once at the end; with the causal mask and
// MQA/GQA head sharing of the FlashRT-HF-kernels page (section "attention
// optimisation"). One work-group per (128-row query tile, head, sequence).
// The causal mask is bottom-right aligned (query i sees key j iff
// j <= i + Skv - Sq), as for the other prefill kernels.
//
// gfx950 mapping:
//   - 4 waves x 32 query rows = a 128-row tile; S^T = K . Q^T and
//     O^T = V^T . P^T on v_mfma_f32_32x32x16_bf16, Q^T held in registers,
//     K read from LDS with ds_read_b128 and V^T with ds_read_b64_tr_b16;
//   - K/V blocks of 64 keys come in by direct-to-LDS loads
//     (buffer_load_dwordx4 ... lds), double-buffered, one barrier per block;
//   - LDS rows are padded to a power-of-two number of 16-byte chunks (8 for
//     d = 32, 16 for d = 96) so the XOR swizzles stay inside the row; the
//     padding chunks are filled with zeros by out-of-range buffer loads;
//   - d = 256 needs O^T (128 registers) and Q^T (64) per wave, so it runs one
//     wave per SIMD with up to 512 registers and 128 KB of LDS per work-group;
//     d = 32 and 96 run two or more work-groups per CU, whose waves overlap
//     each other's MFMA and softmax phases;
//   - d = 256 grids of fewer than two rounds of 128-row tiles (one work-group
//     per CU) run prefill_hd_ks_kernel instead: 64-row tiles whose keys are
//     split between two wave pairs (below).
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kTile = 128;   // query rows per work-group
constexpr int kKN = 64;      // keys per K/V block
constexpr float kTau = 8.0f; // lazy rescale threshold (log2 units)
constexpr int kXcdsHd = 8;
constexpr int kRankMaxBHd = 512;  // sequences ordered by length in every work-group up to this batch
constexpr int kRsrcW3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kPadOff = 0x80000000u;  // an offset past any block: the load returns zeros

constexpr int pow2ceil(int x) { int r = 1; while (r < x) r *= 2; return r; }

template <int D>
struct HdCfg {
  static constexpr int CH = D / 8;                         // 16-byte chunks per K/V row
  static constexpr int RP = CH < 8 ? 8 : pow2ceil(CH);     // chunks per LDS row (padded)
  static constexpr int KS = D / 16;                        // k-steps of S^T
  static constexpr int DB = D / 32;                        // 32-dim blocks of O^T
  static constexpr int NI = kKN * RP / 64 / 4;             // direct-to-LDS loads per wave per block
  static constexpr int STAGE = kKN * RP * 8;               // bf16 elements per LDS stage of K or V
  static constexpr int OCC = D > 128 ? 1 : 2;              // waves per SIMD the registers allow
};

// K rows are read 16 bytes per lane for 32 consecutive rows at one chunk:
// XOR with row mod RP spreads 8 consecutive rows over 8 distinct chunks.
template <int D>
__device__ __forceinline__ int hswz_k(int row) { return row & (HdCfg<D>::RP - 1); }
// V^T transpose reads: each 16-lane group reads 4 consecutive rows x 32
// bytes; an even XOR keeps each 32-byte chunk pair together and places the
// 4 rows in different bank windows.
template <int D>
__device__ __forceinline__ int hswz_v(int row) { return (HdCfg<D>::RP >= 16 ? 4 : 2) * (row & 3); }

__device__ __forceinline__ float hpair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float hpair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 hbf16x2 __attribute__((ext_vector_type(2)));
typedef float hf32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t hpack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((hf32x2){a, b}, hbf16x2));
}

// CACHE: K and V come from a KV cache in the decode layouts (contiguous
// [B, max_len, Hkv, D] or pages of 16 tokens through a block table) with
// Skv = seqlens[b]: the chunked prefill, whose Sq new queries are the last Sq
// cached tokens (bottom-right causal alignment); a row with no visible key
// gives zeros. Each wave's loads of a 64-key block cover exactly its 16 rows,
// one page, read through one buffer resource bounded at the last valid key.
template <int D, bool CACHE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HdCfg<D>::OCC, HdCfg<D>::OCC)))
prefill_hd_kernel(PrefillParams p) {
  using C = HdCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;

  // Work item I: query tile fastest (most keys first when causal), then
  // query head, then sequence; each XCD takes a contiguous range of items,
  // so the query heads of one kv head share that XCD's L2.
  int t, h, b;
  if constexpr (CACHE && C::OCC > 1) {
    // With a cache a tile's cost is its sequence's cached length. The
    // (sequence, kv head) groups are ordered by descending length and dealt
    // whole, round-robin, to the 8 XCDs (each XCD gets an equal mix of long
    // and short sequences, longest first, and keeps a kv head's K/V in one
    // L2); inside a group, tiles by descending causal cost, then heads.
    // (d = 256, one work-group per CU, keeps the plain order below: measured
    // faster there on mixed lengths.)
    const int G = p.Hq / p.Hkv;
    const int per_group = G * p.nT;
    const int xcd = (int)blockIdx.x % kXcdsHd, idx = (int)blockIdx.x / kXcdsHd;
    const int k = xcd + kXcdsHd * (idx / per_group);
    if (k >= p.B * p.Hkv) return;  // past this XCD's groups (uniform)
    const int within = idx % per_group;
    const int r = k / p.Hkv;
    h = (k % p.Hkv) * G + within % G;
    t = p.nT - 1 - within / G;
    // the sequence of length rank r (longest first, ties by index); beyond
    // kRankMaxBHd sequences, index order
    b = r;
    if (p.B <= kRankMaxBHd) {
      int* rank_slot = (int*)sK0;  // not in use yet
      for (int u0 = tid; u0 < p.B; u0 += 256) {
        const int lt = min(max(p.lens[u0], 0), p.max_len);
        int rank = 0;
        for (int u = 0; u < p.B; ++u) {
          const int lu = min(max(p.lens[u], 0), p.max_len);
          rank += (lu > lt || (lu == lt && u < u0)) ? 1 : 0;
        }
        if (rank == r) *rank_slot = u0;
      }
      __syncthreads();
      b = __builtin_amdgcn_readfirstlane(*rank_slot);
      __syncthreads();  // every wave has read the slot before sK0 is loaded
    }
  } else {
    const int W = p.nT * p.Hq * p.B;
    const int L = blockIdx.x;
    const int xcd = L % kXcdsHd, idx = L / kXcdsHd;
    const int qq = W / kXcdsHd, rr = W % kXcdsHd;
    const int I = (xcd < rr) ? xcd * (qq + 1) + idx : rr * (qq + 1) + (xcd - rr) * qq + idx;
    t = p.nT - 1 - I % p.nT;
    h = (I / p.nT) % p.Hq;
    b = I / (p.nT * p.Hq);
  }
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq;
  const int Skv = CACHE ? min(max(p.lens[b], 0), p.max_len) : p.Skv;
  const int off = Skv - Sq;
  const bool causal = p.causal != 0;
  const float c = p.c;

  const int q_last = min(t * kTile + kTile, Sq) - 1;           // last row of the tile
  const int kend = causal ? min(Skv, q_last + off + 1) : Skv;  // keys the tile sees (CACHE: maybe none)
  const int nblk = max(0, (kend + kKN - 1) / kKN);

  const __bf16* kbh = CACHE ? (const __bf16*)p.k : (const __bf16*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* vbh = CACHE ? (const __bf16*)p.v : (const __bf16*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const uint32_t rowstride = CACHE ? (uint32_t)p.Hkv * D * 2u : (uint32_t)D * 2u;
  const __bf16* qbh = (const __bf16*)p.q + ((size_t)b * p.Hq + h) * (size_t)Sq * D;

  // Direct-to-LDS offsets: LDS chunk P of a block holds logical chunk
  // (P % RP) ^ swz(row) of row P / RP; a padding chunk (logical >= CH) gets
  // an out-of-range offset and is written as zeros.
  // (CACHE: wave w's chunks are rows 16 w .. 16 w + 15 of the block, one
  // page; offsets are relative to that page's first row)
  uint32_t koff[C::NI], voff[C::NI];
#pragma unroll
  for (int ii = 0; ii < C::NI; ++ii) {
    const int P = 64 * (wave * C::NI + ii) + lane;
    const int row = P / C::RP, pc = P % C::RP;
    const int lk = pc ^ hswz_k<D>(row), lv = pc ^ hswz_v<D>(row);
    const uint32_t rb = (uint32_t)(CACHE ? (row & 15) : row) * rowstride;
    koff[ii] = lk < C::CH ? rb + (uint32_t)(lk * 16) : kPadOff;
    voff[ii] = lv < C::CH ? rb + (uint32_t)(lv * 16) : kPadOff;
  }
  auto dma = [&](const __bf16* src, __bf16* stage, const uint32_t* offs, int j) __attribute__((always_inline)) {
    const int kv0 = j * kKN;
    __amdgpu_buffer_rsrc_t rs;
    if constexpr (CACHE) {
      const int r0 = kv0 + 16 * wave;
      const int nvalid = max(0, min(16, Skv - r0));
      const char* base = (const char*)src;
      if (nvalid > 0) {
        const long prow = p.bt ? (long)p.bt[(size_t)b * p.pps + r0 / 16] * 16 : (long)b * p.max_len + r0;
        base += ((size_t)prow * p.Hkv + g) * (size_t)(D * 2);
      }
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                             nvalid > 0 ? (nvalid - 1) * (int)rowstride + D * 2 : 0, kRsrcW3);
    } else {
      const int rows = min(kKN, Skv - kv0);
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)kv0 * D), (short)0, rows * D * 2, kRsrcW3);
    }
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + 64 * (wave * C::NI + ii) * 8), 16,
                                               (int)offs[ii], 0, 0, 0);
  };

  // Q^T operand: lane holds Q[row ln][16 ks + 8 hl .. +8] for every k-step;
  // a negative scale is applied by flipping the sign bits (exact).
  const uint32_t qflip = p.neg ? 0x80008000u : 0u;
  const int qrow = t * kTile + wave * 32 + ln;
  bf16x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (qrow < Sq) x = *(const uint4*)(qbh + (size_t)qrow * D + 16 * ks + 8 * hl);
    x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
    qreg[ks] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 O[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) O[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kr0 = ln * (C::RP * 16), kr1 = (32 + ln) * (C::RP * 16);
  const int sw0 = hswz_k<D>(ln), sw1 = hswz_k<D>(32 + ln);
  auto kread = [&](const char* kb, int kr, int sw, int ks) __attribute__((always_inline)) {
    return *(const bf16x8*)(kb + kr + (((2 * ks + hl) ^ sw) << 4));
  };
  // V^T operand: lane (group gg = lane/16, j = lane%16) reads 8 bytes of rows
  // 32 sub + 16 s + 4 hl + j/4 and +8, at dims 32 db + 16 (gg%2) + 4 (j%4).
  const int gg = lane >> 4, jj = lane & 15, dh = gg & 1;
  auto vread = [&](const char* vb, int sub, int s, int db) __attribute__((always_inline)) {
    const int row1 = 32 * sub + 16 * s + 4 * hl + (jj >> 2);
    const int row2 = row1 + 8;
    const int colb = (32 * db + 16 * dh + 4 * (jj & 3)) * 2;
    const char* a1 = vb + row1 * (C::RP * 16) + (((colb >> 4) ^ hswz_v<D>(row1)) << 4) + (colb & 15);
    const char* a2 = vb + row2 * (C::RP * 16) + (((colb >> 4) ^ hswz_v<D>(row2)) << 4) + (colb & 15);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (nblk > 0) {
    dma(kbh, sK0, koff, 0);
    dma(vbh, sV0, voff, 0);
  }
  const int q0 = t * kTile + wave * 32;
  for (int j = 0; j < nblk; ++j) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block j
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads of the other stage are done
    __syncthreads();
    const bool odd = j & 1;
    if (j + 1 < nblk) {
      dma(kbh, odd ? sK0 : sK1, koff, j + 1);
      dma(vbh, odd ? sV0 : sV1, voff, j + 1);
    }
    const int kv0 = j * kKN;
    // a causal block above every row of this wave contributes nothing
    if (causal && kv0 > q0 + 31 + off) continue;
    const char* kb = (const char*)(odd ? sK1 : sK0);
    const char* vb = (const char*)(odd ? sV1 : sV0);

    f32x16 S0 = f32x16{}, S1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kb, kr0, sw0, ks), qreg[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kb, kr1, sw1, ks), qreg[ks], S1, 0, 0, 0);
    }
    // key of register r of sub-tile u is kv0 + 32u + 4hl + 8(r/4) + r%4;
    // visible iff < Skv and (non-causal or) <= query row + off
    const bool full = kv0 + kKN <= Skv && (!causal || kv0 + kKN - 1 <= q0 + off);
    if (!full) {
      const int kb0 = kv0 + 4 * hl;
      int lim = Skv - 1 - kb0;
      if (causal) lim = min(lim, q0 + ln + off - kb0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ko = 8 * (r >> 2) + (r & 3);
        if (ko > lim) S0[r] = -INFINITY;
        if (ko + 32 > lim) S1[r] = -INFINITY;
      }
    }
    // running reference: raised to the block's scaled row maximum when that
    // exceeds it by more than kTau, so every probability stays <= 2^kTau
    float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[r], S1[r]));
    mx = hpair_max(mx);
    const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
    float alpha = 1.f;
    if (cand > m_run + kTau) {
      alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - cand);
      m_run = cand;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 P[2][2];
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(sub ? S1[r] : S0[r], c, -mu));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint4 w;
        w.x = hpack(e[8 * s + 0], e[8 * s + 1]);
        w.y = hpack(e[8 * s + 2], e[8 * s + 3]);
        w.z = hpack(e[8 * s + 4], e[8 * s + 5]);
        w.w = hpack(e[8 * s + 6], e[8 * s + 7]);
        P[sub][s] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          la += e[8 * s + r];
          lb += e[8 * s + r + 1];
        }
      }
    }
    l_run = alpha * l_run + (la + lb);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(vb, sub, s, db), P[sub][s], O[db], 0, 0, 0);
  }

  // normalise and store (rows past Sq are not written; CACHE: a row with no
  // visible key has l = 0 and gives zeros)
  const float lt = hpair_sum(l_run);
  const float inv = CACHE ? (lt > 0.f ? 1.0f / lt : 0.f) : 1.0f / lt;
  if (qrow < Sq) {
    __bf16* dst = (__bf16*)p.o + (((size_t)b * p.Hq + h) * Sq + qrow) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        uint2 w;
        w.x = hpack(O[db][4 * rg + 0] * inv, O[db][4 * rg + 1] * inv);
        w.y = hpack(O[db][4 * rg + 2] * inv, O[db][4 * rg + 3] * inv);
        *(uint2*)(dst + 32 * db + 8 * rg + 4 * hl) = w;
      }
  }
}

// d = 256 with the keys of each tile split between two wave pairs: a
// work-group owns a 64-row query tile; waves 2kh and 2kh+1 own its two 32-row
// halves over the 32-key blocks kh, kh+2, kh+4, ... (kh = 0, 1), and the two
// partial states of each row are merged through LDS at the end. Against one
// wave per 32 rows over all keys this halves the longest chain of blocks in a
// causal grid, and the 64-row tiles (twice as many work-groups, most keys
// first) fill the CUs in two balanced rounds where 128-row tiles made one
// unbalanced round.
constexpr int kTileKs = 64;  // query rows per work-group
constexpr int kKBKs = 32;    // keys per block

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_hd_ks_kernel(PrefillParams p) {
  using C = HdCfg<D>;
  constexpr int STG = kKBKs * C::RP * 8;      // bf16 elements of one 32-key block
  constexpr int NIK = kKBKs * C::RP / 64 / 2; // direct-to-LDS loads per wave per block (two waves share it)
  // [stage][key half]; the merge reuses this memory
  __shared__ __attribute__((aligned(1024))) __bf16 sK[2][2][STG];
  __shared__ __attribute__((aligned(1024))) __bf16 sV[2][2][STG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int rh = wave & 1, kh = wave >> 1;  // row half, key half

  const int nT = (p.Sq + kTileKs - 1) / kTileKs;
  int t, h, b;
  {
    const int W = nT * p.Hq * p.B;
    const int L = blockIdx.x;
    const int xcd = L % kXcdsHd, idx = L / kXcdsHd;
    const int qq = W / kXcdsHd, rr = W % kXcdsHd;
    const int I = (xcd < rr) ? xcd * (qq + 1) + idx : rr * (qq + 1) + (xcd - rr) * qq + idx;
    t = nT - 1 - I % nT;
    h = (I / nT) % p.Hq;
    b = I / (nT * p.Hq);
  }
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq, Skv = p.Skv, off = Skv - Sq;
  const bool causal = p.causal != 0;
  const float c = p.c;
  const int q_last = min(t * kTileKs + kTileKs, Sq) - 1;
  const int kend = causal ? min(Skv, q_last + off + 1) : Skv;
  const int nb = (kend + kKBKs - 1) / kKBKs;  // 32-key blocks the tile sees
  const int iters = (nb + 1) / 2;

  const __bf16* kbh = (const __bf16*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* vbh = (const __bf16*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* qbh = (const __bf16*)p.q + ((size_t)b * p.Hq + h) * (size_t)Sq * D;

  // this wave loads rows 16 rh .. 16 rh + 15 of its key half's blocks
  uint32_t koff[NIK], voff[NIK];
#pragma unroll
  for (int ii = 0; ii < NIK; ++ii) {
    const int P = 64 * (NIK * rh + ii) + lane;
    const int row = P / C::RP, pc = P % C::RP;
    const int lk = pc ^ hswz_k<D>(row), lv = pc ^ hswz_v<D>(row);
    koff[ii] = lk < C::CH ? (uint32_t)(row * D * 2 + lk * 16) : kPadOff;
    voff[ii] = lv < C::CH ? (uint32_t)(row * D * 2 + lv * 16) : kPadOff;
  }
  auto dma = [&](const __bf16* src, __bf16* stage, const uint32_t* offs, int jb) __attribute__((always_inline)) {
    const int kv0 = jb * kKBKs;
    const int rows = min(kKBKs, Skv - kv0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)kv0 * D), (short)0, rows * D * 2, kRsrcW3);
#pragma unroll
    for (int ii = 0; ii < NIK; ++ii)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + 64 * (NIK * rh + ii) * 8), 16,
                                               (int)offs[ii], 0, 0, 0);
  };

  const uint32_t qflip = p.neg ? 0x80008000u : 0u;
  const int q0 = t * kTileKs + rh * 32;
  const int qrow = q0 + ln;
  bf16x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (qrow < Sq) x = *(const uint4*)(qbh + (size_t)qrow * D + 16 * ks + 8 * hl);
    x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
    qreg[ks] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 O[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) O[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kr0 = ln * (C::RP * 16);
  const int sw0 = hswz_k<D>(ln);
  const int gg = lane >> 4, jj = lane & 15, dh = gg & 1;
  auto vread = [&](const char* vb, int s, int db) __attribute__((always_inline)) {
    const int row1 = 16 * s + 4 * hl + (jj >> 2);
    const int row2 = row1 + 8;
    const int colb = (32 * db + 16 * dh + 4 * (jj & 3)) * 2;
    const char* a1 = vb + row1 * (C::RP * 16) + (((colb >> 4) ^ hswz_v<D>(row1)) << 4) + (colb & 15);
    const char* a2 = vb + row2 * (C::RP * 16) + (((colb >> 4) ^ hswz_v<D>(row2)) << 4) + (colb & 15);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (kh < nb) {
    dma(kbh, sK[0][kh], koff, kh);
    dma(vbh, sV[0][kh], voff, kh);
  }
  for (int i = 0; i < iters; ++i) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of its block
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads of the other stage are done
    __syncthreads();
    const int st = i & 1;
    const int jn = 2 * (i + 1) + kh;
    if (jn < nb) {
      dma(kbh, sK[st ^ 1][kh], koff, jn);
      dma(vbh, sV[st ^ 1][kh], voff, jn);
    }
    const int jb = 2 * i + kh;
    const int kv0 = jb * kKBKs;
    if (jb >= nb || (causal && kv0 > q0 + 31 + off)) continue;
    const char* kb = (const char*)sK[st][kh];
    const char* vb = (const char*)sV[st][kh];

    f32x16 S = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kb + kr0 + (((2 * ks + hl) ^ sw0) << 4)),
                                                 qreg[ks], S, 0, 0, 0);
    // key of register r is kv0 + 4hl + 8(r/4) + r%4
    const bool full = kv0 + kKBKs <= Skv && (!causal || kv0 + kKBKs - 1 <= q0 + off);
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
    mx = hpair_max(mx);
    const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
    float alpha = 1.f;
    if (cand > m_run + kTau) {
      alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - cand);
      m_run = cand;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c, -mu));
    bf16x8 P[2];
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 w;
      w.x = hpack(e[8 * s + 0], e[8 * s + 1]);
      w.y = hpack(e[8 * s + 2], e[8 * s + 3]);
      w.z = hpack(e[8 * s + 4], e[8 * s + 5]);
      w.w = hpack(e[8 * s + 6], e[8 * s + 7]);
      P[s] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
      for (int r = 0; r < 8; r += 2) {
        la += e[8 * s + r];
        lb += e[8 * s + r + 1];
      }
    }
    l_run = alpha * l_run + (la + lb);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(vb, s, db), P[s], O[db], 0, 0, 0);
  }

  // merge the key halves: the kh = 1 waves hand (m, l, O) to the kh = 0 waves
  // of the same rows through LDS (the stages are free once every wave is here)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  float4* xo = (float4*)&sK[0][0][0] + rh * (C::DB * 4 * 64);  // 32 KB per row half
  float* xm = (float*)&sV[0][0][0] + rh * 128;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        xo[(db * 4 + rg) * 64 + lane] =
            make_float4(O[db][4 * rg], O[db][4 * rg + 1], O[db][4 * rg + 2], O[db][4 * rg + 3]);
    xm[lane] = m_run;
    xm[64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = xm[lane], l1 = xm[64 + lane];
    const float M = fmaxf(m_run, m1);  // finite: every row sees key 0 in block 0
    const float f0 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    const float f1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    const float lt = hpair_sum(l_run * f0 + l1 * f1);
    const float inv = 1.0f / lt;
    if (qrow < Sq) {
      __bf16* dst = (__bf16*)p.o + (((size_t)b * p.Hq + h) * Sq + qrow) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float4 o1 = xo[(db * 4 + rg) * 64 + lane];
          const float v0 = (O[db][4 * rg + 0] * f0 + o1.x * f1) * inv;
          const float v1 = (O[db][4 * rg + 1] * f0 + o1.y * f1) * inv;
          const float v2 = (O[db][4 * rg + 2] * f0 + o1.z * f1) * inv;
          const float v3 = (O[db][4 * rg + 3] * f0 + o1.w * f1) * inv;
          uint2 w;
          w.x = hpack(v0, v1);
          w.y = hpack(v2, v3);
          *(uint2*)(dst + 32 * db + 8 * rg + 4 * hl) = w;
        }
    }
  }
}

}  // namespace

hipError_t launch_prefill_hd(const PrefillParams& p, int d, hipStream_t stream) {
  const dim3 grid(p.nT * p.Hq * p.B), block(256);
  if (p.lens) {
    // chunked prefill over a KV cache: the one-group kernel, one work-group
    // per (query tile, head, sequence), padded to whole rounds of (sequence,
    // kv head) groups on the 8 XCDs
    // (d = 32, 96: padded to whole rounds of (sequence, kv head) groups on the
    // 8 XCDs, longest sequences first; d = 256: the plain grid)
    const dim3 grid_c(kXcdsHd * ((p.B * p.Hkv + kXcdsHd - 1) / kXcdsHd) * (p.Hq / p.Hkv) * p.nT);
    if (d == 32)
      hipLaunchKernelGGL((prefill_hd_kernel<32, true>), grid_c, block, 0, stream, p);
    else if (d == 96)
      hipLaunchKernelGGL((prefill_hd_kernel<96, true>), grid_c, block, 0, stream, p);
    else if (d == 256)
      hipLaunchKernelGGL((prefill_hd_kernel<256, true>), grid, block, 0, stream, p);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // d = 256 grids of fewer than two rounds of 128-row tiles (one work-group
  // per CU) take the key-split kernel, whose 64-row tiles balance the CUs
  if (d == 32)
    hipLaunchKernelGGL((prefill_hd_kernel<32, false>), grid, block, 0, stream, p);
  else if (d == 96)
    hipLaunchKernelGGL((prefill_hd_kernel<96, false>), grid, block, 0, stream, p);
  else if (d == 256 && p.cus > 0 && (long)p.nT * p.Hq * p.B < 2L * p.cus)
    hipLaunchKernelGGL(prefill_hd_ks_kernel<256>, dim3(((p.Sq + kTileKs - 1) / kTileKs) * p.Hq * p.B), block, 0,
                       stream, p);
  else if (d == 256)
    hipLaunchKernelGGL((prefill_hd_kernel<256, false>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
