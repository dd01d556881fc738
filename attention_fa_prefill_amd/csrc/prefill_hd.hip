// bf16 prefill for the head dims the ping-pong kernel does not provide
// (d = 32, 256): causal or non-causal MQA/GQA attention with an online
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
//   - LDS rows are padded to a power-of-two number of at least 8 16-byte
//     chunks (8 for d = 32) so the XOR swizzles stay inside the row; the
//     padding chunks are filled with zeros by out-of-range buffer loads;
//   - d = 256 needs O^T (128 registers) and Q^T (64) per wave, so it runs one
//     wave per SIMD with up to 512 registers and 128 KB of LDS per work-group;
//   - d = 32 (with or without a cache), and d = 256 prefill without a cache
//     on grids of fewer than two rounds of 128-row tiles (one work-group per
//     CU), run prefill_hd_ks_kernel instead: smaller tiles whose keys are
//     split between two or four groups of waves (below); at d = 32 four or
//     more of its work-groups share a CU and overlap their waves' MFMA and
//     softmax phases.
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
  // waves per SIMD the kernels are compiled for: d = 256 needs all registers;
  // the d = 32 key-split kernel fits at four (80-82 registers), so at least
  // four work-groups share a CU and overlap their softmax and MFMA phases
  static constexpr int OCC = D > 128 ? 1 : (D <= 32 ? 4 : 2);
};

// K rows are read 16 bytes per lane for 32 consecutive rows at one chunk:
// XOR with row mod RP spreads 8 consecutive rows over 8 distinct chunks.
// At d > 128 a wave holds O^T (128 registers) and Q^T (64) and needs more
// than 256 registers. Q^T is only ever an MFMA operand, so it is kept in the
// accumulation registers (the empty asm pins it there at the top of each
// block) and O^T stays in the vector registers, where the rare rescale and
// the epilogue use it; this file is compiled with the MFMA results in vector
// registers (-mllvm -amdgpu-mfma-vgpr-form=1, set by the build). Otherwise
// O^T is copied between the two register files on every block.
template <int D>
__device__ __forceinline__ void pin_q(bf16x8* qreg) {
  if constexpr (D > 128) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+a"(qreg[ks]));
  }
}

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
// Chunked prefill work order: a tile's cost is its sequence's cached length.
// The (sequence, kv head) groups are ordered by descending length and dealt
// whole, round-robin, to the 8 XCDs (each XCD gets an equal mix of long and
// short sequences, longest first, and keeps a kv head's K/V in one L2);
// inside a group, tiles by descending causal cost (nT tiles), then heads.
// Returns false for a work-group past its XCD's groups (uniform). Every
// thread of the work-group calls it (it synchronises when it ranks the
// lengths); `slot` is an int of LDS not yet in use.
__device__ __forceinline__ bool ranked_cache_item(const PrefillParams& p, int nT, int tid, int* slot, int& b, int& h,
                                                  int& t) {
  const int G = p.Hq / p.Hkv;
  const int per_group = G * nT;
  const int xcd = (int)blockIdx.x % kXcdsHd, idx = (int)blockIdx.x / kXcdsHd;
  const int k = xcd + kXcdsHd * (idx / per_group);
  if (k >= p.B * p.Hkv) return false;
  const int within = idx % per_group;
  const int r = k / p.Hkv;
  h = (k % p.Hkv) * G + within % G;
  t = nT - 1 - within / G;
  // the sequence of length rank r (longest first, ties by index); beyond
  // kRankMaxBHd sequences, index order
  b = r;
  if (p.B <= kRankMaxBHd) {
    for (int u0 = tid; u0 < p.B; u0 += 256) {
      const int lt = min(max(p.lens[u0], 0), p.max_len);
      int rank = 0;
      for (int u = 0; u < p.B; ++u) {
        const int lu = min(max(p.lens[u], 0), p.max_len);
        rank += (lu > lt || (lu == lt && u < u0)) ? 1 : 0;
      }
      if (rank == r) *slot = u0;
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(*slot);
    __syncthreads();  // every wave has read the slot before its memory is reused
  }
  return true;
}

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
  {
    // (with a cache too: at d = 256, one work-group per CU, this order measured
    // faster than the longest-first one on mixed lengths)
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
    pin_q<D>(qreg);
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
    {
      // K operands read kPFS MFMAs ahead (MFMA n: k-step n / 2, sub-tile n % 2)
      constexpr int kNS = 2 * C::KS, kPFS = 4;
      auto kop = [&](int n) __attribute__((always_inline)) {
        return (n & 1) ? kread(kb, kr1, sw1, n >> 1) : kread(kb, kr0, sw0, n >> 1);
      };
      bf16x8 kbuf[kPFS];
#pragma unroll
      for (int n = 0; n < kPFS; ++n) kbuf[n] = kop(n);
#pragma unroll
      for (int n = 0; n < kNS; ++n) {
        const bf16x8 a = kbuf[n % kPFS];
        if (n + kPFS < kNS) kbuf[n % kPFS] = kop(n + kPFS);
        if (n & 1)
          S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[n >> 1], S1, 0, 0, 0);
        else
          S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[n >> 1], S0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
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
    {
      // V^T operands read kPFV MFMAs ahead (MFMA n: sub n / (2 DB), s (n / DB) % 2, db n % DB)
      constexpr int kNV = 4 * C::DB, kPFV = 4;
      auto vop = [&](int n) __attribute__((always_inline)) {
        return vread(vb, n / (2 * C::DB), (n / C::DB) & 1, n % C::DB);
      };
      bf16x8 vbuf[kPFV];
#pragma unroll
      for (int n = 0; n < kPFV; ++n) vbuf[n] = vop(n);
#pragma unroll
      for (int n = 0; n < kNV; ++n) {
        const bf16x8 a = vbuf[n % kPFV];
        if (n + kPFV < kNV) vbuf[n % kPFV] = vop(n + kPFV);
        const int db = n % C::DB;
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[n / (2 * C::DB)][(n / C::DB) & 1], O[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
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

// The keys of each tile split between KH wave groups (KH = 2 or 4): a
// work-group of 4 waves owns a 32·(4/KH)-row query tile; wave w owns the
// 32-row part rh = w mod (4/KH) of it over the 32-key blocks kh, kh+KH,
// kh+2KH, ... (kh = w div (4/KH)), and the KH partial states of each row are
// merged through LDS at the end. Against one wave per 32 rows over all keys
// this divides the longest chain of blocks in a causal grid by KH, and the
// smaller tiles (more work-groups, most keys first) balance the CUs.
//   - d = 256 (KH = 2, 64-row tiles): two rounds at one work-group per CU
//     where 128-row tiles made one unbalanced round.
//   - d = 32 (four or more work-groups per CU; also the chunked prefill over a
//     KV cache, CACHE): a block's work is short and a wave's blocks follow
//     each other (load, MFMAs, softmax), so on small causal grids the longest
//     chains set the time: KH = 4 there, four chains a quarter as long;
//     elsewhere KH = 2 (fewer merges, more K/V reuse). Its
//     LDS rows are not padded (64 bytes, 4 chunks): K is swizzled with bits
//     2-3 of the row, so 16 consecutive rows read one chunk each from 16
//     distinct 16-byte bank groups, and the V^T transpose reads of 32 lanes
//     cover 4 whole consecutive rows (256 contiguous bytes) unswizzled.
constexpr int kKBKs = 32;    // keys per block

template <int D, int KH_>
struct KsCfg {
  static constexpr int KH = KH_;                     // key parts
  static constexpr int RH = 4 / KH;                  // 32-row parts of the tile
  static constexpr int TILE = 32 * RH;               // query rows per work-group
  static constexpr int RP = D <= 32 ? HdCfg<D>::CH : HdCfg<D>::RP;  // 16-byte chunks per LDS row
  static constexpr int STG = kKBKs * RP * 8;         // bf16 elements of one 32-key block
  static constexpr int NIK = kKBKs * RP / 64 / RH;   // direct-to-LDS loads per wave per block (RH waves share it)
};
template <int D>
__device__ __forceinline__ int ks_swz_k(int row) { return D <= 32 ? (row >> 2) & 3 : hswz_k<D>(row); }
template <int D>
__device__ __forceinline__ int ks_swz_v(int row) { return D <= 32 ? 0 : hswz_v<D>(row); }

template <int N>
struct StageIdx {
  static constexpr int value = N;
};

template <int D, int KH_, bool CACHE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HdCfg<D>::OCC, HdCfg<D>::OCC)))
prefill_hd_ks_kernel(PrefillParams p) {
  using C = HdCfg<D>;
  using K = KsCfg<D, KH_>;
  static_assert(KH_ == 2 || KH_ == 4, "two or four key parts");
  constexpr int KH = K::KH, RH = K::RH, RP = K::RP, STG = K::STG, NIK = K::NIK;
  static_assert(NIK >= 1 && 64 * NIK * RH == kKBKs * RP, "a block's chunks are split evenly between its waves");
  static_assert((KH - 1) * C::DB * 4 * 64 * RH * 16 <= 2 * KH * STG * 2, "the merge's partial outputs fit in sK0, sK1");
  static_assert((KH - 1) * 128 * RH * 4 <= KH * STG * 2, "the merge's (m, l) fit in sV0");
  // One array per stage ([key part]), and the loop below names the stages at
  // compile time: the compiler then tells a block's operand reads from the
  // direct-to-LDS loads still in flight into the other stage, and does not
  // make the reads wait for them. The merge reuses this memory.
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[KH][STG];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[KH][STG];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[KH][STG];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[KH][STG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int rh = wave % RH, kh = wave / RH;  // row part, key part

  const int nT = (p.Sq + K::TILE - 1) / K::TILE;
  int t, h, b;
  if constexpr (CACHE) {
    if (!ranked_cache_item(p, nT, tid, (int*)&sK0[0][0], b, h, t)) return;
  } else {
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
  const int Sq = p.Sq;
  const int Skv = CACHE ? min(max(p.lens[b], 0), p.max_len) : p.Skv;
  const int off = Skv - Sq;
  const bool causal = p.causal != 0;
  const float c = p.c;
  const int q_last = min(t * K::TILE + K::TILE, Sq) - 1;
  const int kend = causal ? min(Skv, q_last + off + 1) : Skv;  // (CACHE: maybe none)
  const int nb = max(0, (kend + kKBKs - 1) / kKBKs);  // 32-key blocks the tile sees
  const int iters = (nb + KH - 1) / KH;

  const __bf16* kbh = CACHE ? (const __bf16*)p.k : (const __bf16*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* vbh = CACHE ? (const __bf16*)p.v : (const __bf16*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const uint32_t rowstride = CACHE ? (uint32_t)p.Hkv * D * 2u : (uint32_t)D * 2u;
  const __bf16* qbh = (const __bf16*)p.q + ((size_t)b * p.Hq + h) * (size_t)Sq * D;

  // this wave loads rows (32 / RH) rh .. (32 / RH) (rh + 1) - 1 of its key part's blocks
  // (CACHE: offsets relative to the first row of the row's page of 16)
  uint32_t koff[NIK], voff[NIK];
#pragma unroll
  for (int ii = 0; ii < NIK; ++ii) {
    const int P = 64 * (NIK * rh + ii) + lane;
    const int row = P / RP, pc = P % RP;
    const int lk = pc ^ ks_swz_k<D>(row), lv = pc ^ ks_swz_v<D>(row);
    const uint32_t rb = (uint32_t)(CACHE ? (row & 15) : row) * rowstride;
    koff[ii] = lk < C::CH ? rb + (uint32_t)(lk * 16) : kPadOff;
    voff[ii] = lv < C::CH ? rb + (uint32_t)(lv * 16) : kPadOff;
  }
  auto dma = [&](const __bf16* src, __bf16* stage, const uint32_t* offs, int jb) __attribute__((always_inline)) {
    const int kv0 = jb * kKBKs;
    if constexpr (CACHE) {
      // a load covers RPL rows, LPP loads one page of 16: one buffer
      // resource per page, its record count ending after the last key that
      // exists (rows past it read as zero; a page past the sequence is
      // neither looked up in the block table nor read)
      constexpr int RPL = 64 / RP, LPP = 16 / RPL;
      static_assert(RPL <= 16 && NIK % LPP == 0, "a wave's loads cover whole pages");
#pragma unroll
      for (int pg = 0; pg < NIK / LPP; ++pg) {
        const int r0 = kv0 + RPL * (NIK * rh + pg * LPP);  // first row of the page
        const int nvalid = max(0, min(16, Skv - r0));
        const char* base = (const char*)src;
        if (nvalid > 0) {
          const long prow = p.bt ? (long)p.bt[(size_t)b * p.pps + r0 / 16] * 16 : (long)b * p.max_len + r0;
          base += ((size_t)prow * p.Hkv + g) * (size_t)(D * 2);
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)base, (short)0, nvalid > 0 ? (nvalid - 1) * (int)rowstride + D * 2 : 0, kRsrcW3);
#pragma unroll
        for (int jj = 0; jj < LPP; ++jj) {
          const int ii = pg * LPP + jj;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + 64 * (NIK * rh + ii) * 8), 16,
                                                   (int)offs[ii], 0, 0, 0);
        }
      }
    } else {
      const int rows = min(kKBKs, Skv - kv0);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)kv0 * D), (short)0, rows * D * 2, kRsrcW3);
#pragma unroll
      for (int ii = 0; ii < NIK; ++ii)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + 64 * (NIK * rh + ii) * 8), 16,
                                                 (int)offs[ii], 0, 0, 0);
    }
  };

  const uint32_t qflip = p.neg ? 0x80008000u : 0u;
  const int q0 = t * K::TILE + rh * 32;
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

  const int kr0 = ln * (RP * 16);
  const int sw0 = ks_swz_k<D>(ln);
  const int gg = lane >> 4, jj = lane & 15, dh = gg & 1;
  auto vread = [&](const char* vb, int s, int db) __attribute__((always_inline)) {
    const int row1 = 16 * s + 4 * hl + (jj >> 2);
    const int row2 = row1 + 8;
    const int colb = (32 * db + 16 * dh + 4 * (jj & 3)) * 2;
    const char* a1 = vb + row1 * (RP * 16) + (((colb >> 4) ^ ks_swz_v<D>(row1)) << 4) + (colb & 15);
    const char* a2 = vb + row2 * (RP * 16) + (((colb >> 4) ^ ks_swz_v<D>(row2)) << 4) + (colb & 15);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (kh < nb) {
    dma(kbh, sK0[kh], koff, kh);
    dma(vbh, sV0[kh], voff, kh);
  }
  auto step = [&](auto stage, int i) __attribute__((always_inline)) {
    constexpr int st = decltype(stage)::value;
    auto& kcur = st ? sK1 : sK0;
    auto& vcur = st ? sV1 : sV0;
    auto& knxt = st ? sK0 : sK1;
    auto& vnxt = st ? sV0 : sV1;
    pin_q<D>(qreg);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of its block
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads of the other stage are done
    // With one row part (RH = 1) each wave loads and reads only its own key
    // part's stages, so its own waits above order everything and the key
    // parts run their chains without meeting; waves that share a block (RH =
    // 2) meet here.
    if constexpr (RH > 1) __syncthreads();
    const int jn = KH * (i + 1) + kh;
    const int jb = KH * i + kh;
    const int kv0 = jb * kKBKs;
    const bool live = !(jb >= nb || (causal && kv0 > q0 + 31 + off));
    const char* kb = (const char*)kcur[kh];
    const char* vb = (const char*)vcur[kh];
    // The compiler cannot tell a V^T transpose read from the loads in flight
    // into the other stage and would make it wait for them: at d = 32 the
    // block's V^T operands (8 registers) are therefore read before the next
    // block's loads are issued.
    constexpr int kNV = 2 * C::DB;
    constexpr bool kVFirst = D <= 32;
    bf16x8 vpre[kVFirst ? kNV : 1];
    if constexpr (kVFirst) {
      if (live) {
#pragma unroll
        for (int n = 0; n < kNV; ++n) vpre[n] = vread(vb, n / C::DB, n % C::DB);
      }
    }
    if (jn < nb) {
      dma(kbh, knxt[kh], koff, jn);
      dma(vbh, vnxt[kh], voff, jn);
    }
    if (!live) return;
    f32x16 S = f32x16{};
    {
      // K operands read kPFS k-steps ahead
      constexpr int kPFS = C::KS < 4 ? C::KS : 4;
      auto kop = [&](int ks) __attribute__((always_inline)) {
        return *(const bf16x8*)(kb + kr0 + (((2 * ks + hl) ^ sw0) << 4));
      };
      bf16x8 kbuf[kPFS];
#pragma unroll
      for (int n = 0; n < kPFS; ++n) kbuf[n] = kop(n);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = kbuf[ks % kPFS];
        if (ks + kPFS < C::KS) kbuf[ks % kPFS] = kop(ks + kPFS);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], S, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
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
    // The block is exponentiated against the current reference without a
    // max search; the block's maximum is taken (and the reference raised when
    // it grows by more than kTau) only when a row has no reference yet, or
    // when a lane's partial block sum passes 2^16 (which also catches inf and
    // NaN). Probabilities therefore stay at most 2^16.
    float alpha = 1.f;
    float e[16];
    float la = 0.f, lb = 0.f;
    auto exponentiate = [&](float mu) __attribute__((always_inline)) {
      la = 0.f;
      lb = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c, -mu));
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        la += e[r];
        lb += e[r + 1];
      }
    };
    bool redo = __any(m_run == -INFINITY);
    if (!redo) {
      exponentiate(m_run);
      redo = __any(!(la + lb <= 65536.f));
    }
    if (redo) {
      float mx = S[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
      mx = hpair_max(mx);
      const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
      if (cand > m_run + kTau) {
        alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - cand);
        m_run = cand;
      }
      exponentiate((m_run == -INFINITY) ? 0.f : m_run);
    }
    bf16x8 P[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 w;
      w.x = hpack(e[8 * s + 0], e[8 * s + 1]);
      w.y = hpack(e[8 * s + 2], e[8 * s + 3]);
      w.z = hpack(e[8 * s + 4], e[8 * s + 5]);
      w.w = hpack(e[8 * s + 6], e[8 * s + 7]);
      P[s] = __builtin_bit_cast(bf16x8, w);
    }
    l_run = alpha * l_run + (la + lb);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    if constexpr (kVFirst) {
#pragma unroll
      for (int n = 0; n < kNV; ++n) {
        const int db = n % C::DB;
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vpre[n], P[n / C::DB], O[db], 0, 0, 0);
      }
    } else {
      // V^T operands read kPFV MFMAs ahead (MFMA n: s n / DB, db n % DB)
      constexpr int kPFV = kNV < 4 ? kNV : 4;
      bf16x8 vbuf[kPFV];
#pragma unroll
      for (int n = 0; n < kPFV; ++n) vbuf[n] = vread(vb, n / C::DB, n % C::DB);
#pragma unroll
      for (int n = 0; n < kNV; ++n) {
        const bf16x8 a = vbuf[n % kPFV];
        if (n + kPFV < kNV) vbuf[n % kPFV] = vread(vb, (n + kPFV) / C::DB, (n + kPFV) % C::DB);
        const int db = n % C::DB;
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[n / C::DB], O[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int i = 0; i < iters; i += 2) {
    step(StageIdx<0>{}, i);
    if (i + 1 < iters) step(StageIdx<1>{}, i + 1);
  }

  // merge the key parts: the kh > 0 waves hand (m, l, O) to the kh = 0 wave
  // of the same rows through LDS (the stages are free once every wave is here)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // O: [key part - 1][row part][db][rg][lane] in float4s over sK0, then sK1
  // (KX float4s each, a multiple of 64, so a wave's 64 never straddle them)
  constexpr int KX = KH * STG / 8;
  static_assert(KX % 64 == 0, "a wave's float4s lie in one array");
  auto xo = [&](int f) __attribute__((always_inline)) {
    return f < KX ? (float4*)&sK0[0][0] + f : (float4*)&sK1[0][0] + (f - KX);
  };
  float* xm = (float*)&sV0[0][0];  // [key part - 1][row part][m, l][lane]
  constexpr int XO = RH * C::DB * 4 * 64, XM = RH * 128;
  if (kh > 0) {
    const int xw = (kh - 1) * XO + rh * (C::DB * 4 * 64);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *xo(xw + (db * 4 + rg) * 64 + lane) =
            make_float4(O[db][4 * rg], O[db][4 * rg + 1], O[db][4 * rg + 2], O[db][4 * rg + 3]);
    float* xmw = xm + (kh - 1) * XM + rh * 128;
    xmw[lane] = m_run;
    xmw[64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 0) {
    float mk[KH], lk[KH], f[KH];
    mk[0] = m_run;
    lk[0] = l_run;
#pragma unroll
    for (int u = 1; u < KH; ++u) {
      mk[u] = xm[(u - 1) * XM + rh * 128 + lane];
      lk[u] = xm[(u - 1) * XM + rh * 128 + 64 + lane];
    }
    float M = mk[0];  // finite unless the row sees no key (CACHE, Skv < Sq)
#pragma unroll
    for (int u = 1; u < KH; ++u) M = fmaxf(M, mk[u]);
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < KH; ++u) {
      f[u] = (mk[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk[u] - M);
      lsum += lk[u] * f[u];
    }
    const float lt = hpair_sum(lsum);
    // (CACHE: a row with no visible key has l = 0 and gives zeros)
    const float inv = CACHE ? (lt > 0.f ? 1.0f / lt : 0.f) : 1.0f / lt;
    if (qrow < Sq) {
      __bf16* dst = (__bf16*)p.o + (((size_t)b * p.Hq + h) * Sq + qrow) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          float v0 = O[db][4 * rg + 0] * f[0], v1 = O[db][4 * rg + 1] * f[0];
          float v2 = O[db][4 * rg + 2] * f[0], v3 = O[db][4 * rg + 3] * f[0];
#pragma unroll
          for (int u = 1; u < KH; ++u) {
            const float4 o1 = *xo((u - 1) * XO + rh * (C::DB * 4 * 64) + (db * 4 + rg) * 64 + lane);
            v0 += o1.x * f[u];
            v1 += o1.y * f[u];
            v2 += o1.z * f[u];
            v3 += o1.w * f[u];
          }
          uint2 w;
          w.x = hpack(v0 * inv, v1 * inv);
          w.y = hpack(v2 * inv, v3 * inv);
          *(uint2*)(dst + 32 * db + 8 * rg + 4 * hl) = w;
        }
    }
  }
}

}  // namespace

hipError_t launch_prefill_hd(const PrefillParams& p, int d, hipStream_t stream) {
  const dim3 grid(p.nT * p.Hq * p.B), block(256);
  if (p.lens) {
    // chunked prefill over a KV cache: at d = 32 the key-split kernel, one
    // work-group per (query tile, head, sequence), padded to whole rounds of
    // (sequence, kv head) groups on the 8 XCDs, longest sequences first; at
    // d = 256 the one-group kernel in the plain order (the key-split kernel
    // measured 1-2 % slower there)
    const long groups = (long)kXcdsHd * ((p.B * p.Hkv + kXcdsHd - 1) / kXcdsHd) * (p.Hq / p.Hkv);
    const long tiles64c = (long)((p.Sq + 63) / 64) * p.Hq * p.B;
    if (d == 32 && p.causal && p.cus > 0 && tiles64c <= 8L * p.cus)
      return launch_kernel(prefill_hd_ks_kernel<32, 4, true>, dim3(groups * ((p.Sq + 31) / 32)), block, stream, p);
    else if (d == 32)
      return launch_kernel(prefill_hd_ks_kernel<32, 2, true>, dim3(groups * ((p.Sq + 63) / 64)), block, stream, p);
    else if (d == 256)
      return launch_kernel(prefill_hd_kernel<256, true>, grid, block, stream, p);
    else
      return hipErrorInvalidValue;
  }
  // d = 32 takes the key-split kernel; d = 256 takes it on causal grids of
  // fewer than two rounds of 128-row tiles (one work-group per CU) with at
  // least 10 tiles per head, where the one-group kernel's longest tile would
  // set the time (measured: key-split faster from 12 tiles per head, the
  // one-group kernel from 8 tiles down and on every non-causal grid)
  const long tiles64 = (long)((p.Sq + 63) / 64) * p.Hq * p.B;
  const dim3 grid_ks2(tiles64), grid_ks4(((p.Sq + 31) / 32) * p.Hq * p.B);
  // d = 32: four key parts on causal grids of at most two rounds of 64-row
  // tiles (four work-groups per CU), two otherwise
  if (d == 32 && p.causal && p.cus > 0 && tiles64 <= 8L * p.cus)
    return launch_kernel(prefill_hd_ks_kernel<32, 4, false>, grid_ks4, block, stream, p);
  else if (d == 32)
    return launch_kernel(prefill_hd_ks_kernel<32, 2, false>, grid_ks2, block, stream, p);
  else if (d == 256 && p.causal && p.nT >= 10 && p.cus > 0 && (long)p.nT * p.Hq * p.B < 2L * p.cus)
    return launch_kernel(prefill_hd_ks_kernel<256, 2, false>, grid_ks2, block, stream, p);
  else if (d == 256)
    return launch_kernel(prefill_hd_kernel<256, false>, grid, block, stream, p);
  else
    return hipErrorInvalidValue;
}

}  // namespace fa
