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
//   - work-groups are ordered so that all query heads sharing a kv head run on
//     one XCD (work-group L runs on XCD L % 8): each K/V block is fetched from
//     HBM into one L2 and reused there.
//   - K/V blocks of 64 keys go HBM/L2 -> LDS with 16-byte direct-to-LDS buffer
//     loads, double-buffered per group, issued two slots ahead of their use.
//   - The KV-cache variant (chunked prefill) reads K/V pages of 16 tokens from
//     a contiguous or paged cache, one buffer resource per page, and gives each
//     work-group one tile; the (sequence, kv head) groups are ordered by
//     descending cached length (see the kernel's template comment).
//
// Per wave and per 64-key block (two 32-key sub-tiles):
//   S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T held
//   in VGPRs), so each lane holds 16 scores of one query; the row max needs only
//   an in-lane max and one v_permlane32_swap with the other half-wave.
//   P = exp2(S*c - m) with c = scale*log2(e). m is an exponent reference, not
//   necessarily the exact running max: a block is exponentiated against the
//   current m without a max search, and the max is taken (m raised by more
//   than kTau, O and l rescaled, block redone) only when a row has no
//   reference yet or its block sum exceeds kRedo. Any reference gives the same
//   normalised result in exact arithmetic.
//   O^T += V^T . P^T on the same MFMA: A = V^T read with ds_read_b64_tr_b16
//   from the row-major V tile in LDS, B = P^T straight from the score registers
//   (the contraction order over keys is permuted to match their lane layout).
//
// Ping-pong schedule. A wave alternates two kinds of slot: an MFMA slot
// M(k) = { O += V(k-1)^T P(k-1)^T ; S(k) = K(k) Q^T } and a vector slot
// V(k) = { softmax of S(k) -> P(k) }. Group B runs half an iteration behind
// group A, and the groups swap slot kinds at every barrier, so on each SIMD one
// wave issues MFMA while the other issues the softmax. The barriers only order
// LDS (no wait for outstanding HBM loads): a group waits for its own
// direct-to-LDS loads right before the barrier that opens its next MFMA slot.
// The K loads of block k+1 are issued one at a time between the MFMAs of
// M(k), the V loads of block k at the start of V(k); the wave in its MFMA
// slot runs at raised issue priority (s_setprio 1).
//
// Head dims 64, 96 and 128. An LDS row holds a power-of-two number of 16-byte
// chunks so that the XOR swizzles stay inside it: d = 96 rows (12 chunks) are
// padded to 16, and the direct-to-LDS lanes that land on padding chunks get
// an out-of-range buffer offset, so they read nothing and write zeros.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 128;     // query rows per wave group
constexpr int kBN = 64;      // keys per KV block
constexpr float kTau = 8.0f; // lazy rescale threshold (log2 units)
constexpr float kRedo = 65536.0f;  // partial row sum above which a block is redone with its maximum
constexpr int kXcds = 8;
constexpr int kRankMaxB = 512;  // sequences ordered by length in every work-group up to this batch     // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

constexpr uint32_t kPadOff = 0x80000000u;  // a buffer offset past any block: the load returns zeros

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;               // 16-byte chunks per K/V row
  static constexpr int RP = D == 96 ? 16 : CH;   // chunks per LDS row (padded to a power of two)
  static constexpr int RB = RP * 16;             // bytes per LDS row
  static constexpr int ELEMS = kBN * RP * 8;     // bf16 elements per K or V block in LDS
  static constexpr int NI = kBN * RP / 64 / 4;   // direct-to-LDS loads per wave per block
  static constexpr int KS = D / 16;              // k-steps of S^T = K . Q^T
  static constexpr int DB = D / 32;              // 32-row d blocks of O^T
  static constexpr int XO = 64 * DB * 16;        // floats of one wave's O^T in the exchange
};

// LDS swizzles (16-byte chunk index XOR a function of the row).
// K (and staged Q) rows are read 16 bytes per lane for 16 consecutive rows at
// one chunk: XOR with row mod RP spreads them over all banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (Cfg<D>::RP - 1); }
// V is read by transpose reads: each 16-lane group touches 4 consecutive rows x
// 32 bytes. XOR with 2*(row%4) (8-chunk rows) / 4*(row%4) (16-chunk rows)
// places those 4 rows in different bank windows and keeps each 32-byte pair of
// chunks together.
template <int D>
__device__ __forceinline__ int swz_v(int row) { return (Cfg<D>::RP >= 16 ? 4 : 2) * (row & 3); }

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

// Barrier that orders LDS only: the wave's LDS reads are complete before it
// arrives; outstanding HBM loads are not waited for (the caller waits for its
// own direct-to-LDS loads where their data is needed). The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// CACHE: K and V come from a KV cache in the decode layouts (contiguous
// [B, max_len, Hkv, D] or pages of 16 tokens [pages, 16, Hkv, D] through a
// block table) with Skv = seqlens[b] per sequence: the chunked prefill of a
// serving loop, whose Sq new queries are the last Sq of the Skv cached tokens
// (bottom-right causal alignment). A query row with no visible key (causal,
// Skv < Sq) gives zeros.
template <int D, bool CACHE>
__global__ void __launch_bounds__(512) prefill_bf16_kernel(PrefillParams p) {
  using C = Cfg<D>;
  // Two stages x {K, V}, each holding both groups' blocks, plus a staging area
  // for the second query tile of group A. Separate arrays let the compiler see
  // that a block being loaded never aliases the block being read.
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[2 * C::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 sQ[kBM * C::RP * 8];

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: keep it (and everything derived
  // from it) in scalar registers so that per-wave decisions are scalar branches.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0 = group A, 1 = group B
  const int wg = wave & 3;    // wave within group
  const int hl = lane >> 5;   // half-wave
  const int ln = lane & 31;
  // XCD-aware work order: work item I (pair fastest, then query head, then
  // batch) goes to the work-group that puts contiguous item ranges on one XCD.
  int pidx, h, b;
  if constexpr (CACHE) {
    // One query tile per work-group (both groups split its keys, as for the
    // middle tile of an odd tile count): with a cache the tiles of a sequence
    // cost about the same, and the cost is its cached length, which differs
    // between sequences. The (sequence, kv head) groups are ordered by
    // descending cached length and dealt round-robin to the 8 XCDs, whole, so
    // each XCD gets an equal mix of long and short sequences, runs its longest
    // work first, and keeps a kv head's K/V in one L2.
    const int G = p.Hq / p.Hkv;
    const int per_group = G * p.nT;
    const int xcd = (int)blockIdx.x % kXcds, idx = (int)blockIdx.x / kXcds;
    const int k = xcd + kXcds * (idx / per_group);
    if (k >= p.B * p.Hkv) return;  // past this XCD's groups (uniform)
    const int within = idx % per_group;
    const int r = k / p.Hkv;
    // inside a group, tiles by descending (causal) cost, then heads
    h = (k % p.Hkv) * G + within % G;
    pidx = p.nT - 1 - within / G;
    // the sequence of length rank r (longest first, ties by index); beyond
    // kRankMaxB sequences, index order
    b = r;
    if (p.B <= kRankMaxB) {
      int* rank_slot = (int*)sQ;  // sQ is not in use yet
      if (tid < p.B) {
        const int lt = min(max(p.lens[tid], 0), p.max_len);
        int rank = 0;
        for (int u = 0; u < p.B; ++u) {
          const int lu = min(max(p.lens[u], 0), p.max_len);
          rank += (lu > lt || (lu == lt && u < tid)) ? 1 : 0;
        }
        if (rank == r) *rank_slot = tid;
      }
      __syncthreads();
      b = __builtin_amdgcn_readfirstlane(*rank_slot);
      __syncthreads();  // every wave has read the slot before sQ is reused
    }
  } else {
    const int W = p.nP * p.Hq * p.B;
    const int L = blockIdx.x;
    const int xcd = L % kXcds, idx = L / kXcds;
    const int q = W / kXcds, r = W % kXcds;
    const int I = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    pidx = I % p.nP;
    h = (I / p.nP) % p.Hq;
    b = I / (p.nP * p.Hq);
  }
  const int g = (int)((long)h * p.Hkv / p.Hq);
  const int Sq = p.Sq;
  const int Skv = CACHE ? min(max(p.lens[b], 0), p.max_len) : p.Skv;
  const int off = Skv - Sq;
  const bool causal = p.causal != 0;
  const float c = p.c;

  auto nblocks = [&](int t) __attribute__((always_inline)) {
    const int end = causal ? min(Skv, (t + 1) * kBM + off) : Skv;
    const int n = (end + kBN - 1) / kBN;
    return CACHE ? max(0, n) : n;  // (CACHE: a causal tile above every key has none)
  };
  const int t0 = pidx, t1 = CACHE ? pidx : p.nT - 1 - pidx;
  const int n1 = nblocks(t1);
  const int nA0 = (t0 == t1) ? 0 : nblocks(t0);
  const int jB = min(n1, (nA0 + n1 + 1) / 2);  // group B: t1 blocks [0, jB)
  const int cntA = nA0 + (n1 - jB), cntB = jB;
  const bool split = jB < n1;                  // group A holds a partial of t1
  const int cnt = grp ? cntB : cntA;
  auto kv_of = [&](int i) __attribute__((always_inline)) { return grp ? i : (i < nA0 ? i : jB + (i - nA0)); };
  auto tile_of = [&](int i) __attribute__((always_inline)) { return grp ? t1 : (i < nA0 ? t0 : t1); };

  const __bf16* kbh = CACHE ? (const __bf16*)p.k : (const __bf16*)p.k + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* vbh = CACHE ? (const __bf16*)p.v : (const __bf16*)p.v + ((size_t)b * p.Hkv + g) * (size_t)Skv * D;
  const __bf16* qbh = (const __bf16*)p.q + ((size_t)b * p.Hq + h) * (size_t)Sq * D;

  // Per-lane byte offsets (inside a 64-key block) of this lane's direct-to-LDS
  // loads: LDS chunk P of the block holds logical chunk (P % RP) ^ swz(row) of
  // row P / RP; a padding chunk (logical >= CH, D = 96) gets an out-of-range
  // offset and is written as zeros.
  // (CACHE: wave wg's loads of a block cover exactly its 16 rows 16 wg ..
  // 16 wg + 15, one page, and rows are rowstride bytes apart.)
  static_assert(64 * C::NI / C::RP == 16, "one page of rows per wave and block");
  const uint32_t rowstride = CACHE ? (uint32_t)p.Hkv * D * 2u : (uint32_t)D * 2u;
  uint32_t koff[C::NI], voff[C::NI];
#pragma unroll
  for (int ii = 0; ii < C::NI; ++ii) {
    const int P = 64 * (wg * C::NI + ii) + lane;
    const int row = P / C::RP, pc = P % C::RP;
    const int lk = pc ^ swz_k<D>(row), lv = pc ^ swz_v<D>(row);
    const uint32_t rbase = (uint32_t)(CACHE ? (row & 15) : row) * rowstride;
    koff[ii] = lk < C::CH ? rbase + (uint32_t)(lk << 4) : kPadOff;
    voff[ii] = lv < C::CH ? rbase + (uint32_t)(lv << 4) : kPadOff;
  }
  // CACHE: buffer resource over this wave's page of block j of the K (or V)
  // cache; its record count ends after the last key that exists, so rows past
  // Skv read as zero, and a page past the sequence is neither looked up in the
  // block table nor read.
  // The cache row of the page comes from page_row, looked up ahead of the
  // loads (a scalar load waited for next to the loads would stall the MFMA
  // stream once per load).
  auto page_row = [&](int j, bool valid) __attribute__((always_inline)) {
    const int r0 = j * kBN + 16 * wg;
    if (!CACHE || !valid || r0 >= Skv) return (long)-1;
    return p.bt ? (long)p.bt[(size_t)b * p.pps + r0 / 16] * 16 : (long)b * p.max_len + r0;
  };
  auto page_rsrc = [&](const __bf16* cache, int j, long prow) __attribute__((always_inline)) {
    const int r0 = j * kBN + 16 * wg;
    const int nvalid = prow >= 0 ? max(0, min(16, Skv - r0)) : 0;
    const char* base = (const char*)cache;
    if (nvalid > 0) base += ((size_t)prow * p.Hkv + g) * (size_t)(D * 2);
    const int nrec = nvalid > 0 ? (nvalid - 1) * (int)rowstride + D * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, kRsrcWord3);
  };
  // One K or V block -> this group's slot of an LDS stage. The buffer resource
  // covers only the keys that exist, so rows past Skv read as zero.
  auto dma_one = [&](const __bf16* src_bh, __bf16* stage, const uint32_t* offs, int j, bool valid, int ii, long prow) __attribute__((always_inline)) {
    const int kv0 = j * kBN;
    const int rows = valid ? min(kBN, Skv - kv0) : 0;
    const __amdgpu_buffer_rsrc_t rs = CACHE ? page_rsrc(src_bh, j, prow) : __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src_bh + (size_t)(valid ? kv0 : 0) * D), (short)0, rows * D * 2, kRsrcWord3);
    __bf16* dst0 = stage + grp * C::ELEMS;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst0 + 64 * (wg * C::NI + ii) * 8), 16, (int)offs[ii], 0,
                                             0, 0);
  };
  auto dma = [&](const __bf16* src_bh, __bf16* stage, const uint32_t* offs, int j) __attribute__((always_inline)) {
    const int kv0 = j * kBN;
    const int rows = min(kBN, Skv - kv0);
    const __amdgpu_buffer_rsrc_t rs = CACHE ? page_rsrc(src_bh, j, page_row(j, true)) :
        __builtin_amdgcn_make_buffer_rsrc((void*)(src_bh + (size_t)kv0 * D), (short)0, rows * D * 2, kRsrcWord3);
    __bf16* dst0 = stage + grp * C::ELEMS;
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst0 + 64 * (wg * C::NI + ii) * 8), 16,
                                               (int)offs[ii], 0, 0, 0);
  };

  f32x16 O[C::DB];
  bf16x8 qreg[C::KS];
  float m_run = -INFINITY, l_run = 0.f;
  int cur_tile = -1;

  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[db][r] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };

  const uint32_t qflip = p.neg ? 0x80008000u : 0u;
  // Q^T operand: lane holds Q[row ln][16 ks + 8 hl .. +8] for every k-step.
  auto load_q_global = [&](int t) __attribute__((always_inline)) {
    const int row = t * kBM + wg * 32 + ln;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < Sq) x = *(const uint4*)(qbh + (size_t)row * D + 16 * ks + 8 * hl);
      x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  };
  // Group A needs its second tile's Q (tile t1) at the tile switch; group B
  // holds exactly those rows in registers (its only tile is t1), so each B
  // wave writes them to LDS in the prologue, in the layout load_q_lds reads
  // (the same lane owns the same 16 bytes on both sides), without the sign
  // flip. No second read of Q from memory.
  auto share_q = [&]() __attribute__((always_inline)) {
    const int row = wg * 32 + ln;
    char* base = (char*)sQ + row * C::RB;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 x = __builtin_bit_cast(uint4, qreg[ks]);
      x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
      *(uint4*)(base + (((2 * ks + hl) ^ swz_k<D>(row)) << 4)) = x;
    }
  };
  auto load_q_lds = [&]() __attribute__((always_inline)) {
    const int row = wg * 32 + ln;
    const char* base = (const char*)sQ + row * C::RB;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 x = *(const uint4*)(base + (((2 * ks + hl) ^ swz_k<D>(row)) << 4));
      x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  };

  auto store_tile = [&](int t) __attribute__((always_inline)) {
    const float lt = pair_sum(l_run);
    // (CACHE: a row with no visible key has l = 0 and gives zeros)
    const float inv = CACHE ? (lt > 0.f ? 1.0f / lt : 0.f) : 1.0f / lt;
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

  const int kr0 = ln * C::RB, kr1 = (32 + ln) * C::RB;
  const int sw0 = swz_k<D>(ln), sw1 = swz_k<D>(32 + ln);
  auto kread = [&](const char* kbase, int kr, int sw, int ks) __attribute__((always_inline)) {
    return *(const bf16x8*)(kbase + kr + (((2 * ks + hl) ^ sw) << 4));
  };
  // V^T operand (transpose reads): lane (group gg = lane/16, j = lane%16) reads
  // 8 bytes of row (32 sub + 16 s + 4 hl + j/4 [+8]) at dims 32 db + 16 (gg%2) + 4 (j%4).
  const int gg = lane >> 4, jj = lane & 15, dh = gg & 1;
  auto vread = [&](const char* vbase, int sub, int s, int db) __attribute__((always_inline)) {
    const int row1 = 32 * sub + 16 * s + 4 * hl + (jj >> 2);
    const int row2 = row1 + 8;
    const int colb = (32 * db + 16 * dh + 4 * (jj & 3)) * 2;
    const char* a1 = vbase + row1 * C::RB + (((colb >> 4) ^ swz_v<D>(row1)) << 4) + (colb & 15);
    const char* a2 = vbase + row2 * C::RB + (((colb >> 4) ^ swz_v<D>(row2)) << 4) + (colb & 15);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- slot state carried between slots
  f32x16 S0 = f32x16{}, S1 = f32x16{};  // scores of the block in flight (M -> V slot)
  bf16x8 P[2][2];                        // probabilities (V -> next M slot)
  bool s_vis = false;                    // scores in S0/S1 belong to a block this wave sees
  bool p_vis = false;                    // P holds a block to accumulate
  int s_kv0 = 0, s_q0 = 0;               // key / query origin of the block in S0/S1

  // MFMA slot k: PV of block k-1, tile switch if block k starts a new tile,
  // then S of block k. (sKc: K stage of block k; sVp: V stage of block k-1;
  // sKn: stage that receives K of block k+1.)
  // It runs as one stream of 32 MFMAs - 16 of PV, then 16 of S - whose LDS
  // operands are read kPF MFMAs ahead, so the matrix core does not wait on LDS
  // latency. When no PV is pending its probabilities are zero (the V stage
  // always holds finite data); when block k is not needed its scores are
  // computed and dropped. Both cases are rare, and branch-free this way.
  constexpr int kPV = 4 * C::DB;  // PV MFMAs: (sub, s, db)
  constexpr int kS = 2 * C::KS;   // S MFMAs: (ks, sub)
  constexpr int kPF = 4;          // operand prefetch distance (MFMAs)
  auto mslot = [&](int k, const __bf16* sKc, const __bf16* sVp, __bf16* sKn) __attribute__((always_inline)) {
    const char* vbase = (const char*)(sVp + grp * C::ELEMS);
    const char* kbase = (const char*)(sKc + grp * C::ELEMS);
    if (!p_vis) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      P[0][0] = P[0][1] = P[1][0] = P[1][1] = __builtin_bit_cast(bf16x8, z);
    }
    S0 = f32x16{};
    S1 = f32x16{};
    // operand of MFMA number i of the stream
    auto opnd = [&](int i) __attribute__((always_inline)) {
      if (i < kPV) return vread(vbase, i / (2 * C::DB), (i / C::DB) & 1, i % C::DB);
      const int j = i - kPV;
      return kread(kbase, (j & 1) ? kr1 : kr0, (j & 1) ? sw1 : sw0, j >> 1);
    };
    // (CACHE: this wave's page row of K(k+1), looked up first)
    const long prk = page_row(kv_of(k + 1), k + 1 < cnt);
    bf16x8 buf[kPF];
#pragma unroll
    for (int i = 0; i < kPF; ++i) buf[i] = opnd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPV + kS; ++i) {
      const bf16x8 a = buf[i % kPF];
      if (i + kPF < kPV + kS) buf[i % kPF] = opnd(i + kPF);
      if (i >= kPV && i < kPV + 2 * C::NI && ((i - kPV) & 1) == 0) {
        // one direct-to-LDS load between every other MFMA: K of block k+1
        const int n = (i - kPV) >> 1;
        dma_one(kbh, sKn, koff, kv_of(k + 1), k + 1 < cnt, n, prk);
      }
      if (i < kPV) {
        const int sub = i / (2 * C::DB), ss = (i / C::DB) & 1, db = i % C::DB;
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[sub][ss], O[db], 0, 0, 0);
      } else {
        const int j = i - kPV;
        if (j & 1)
          S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[j >> 1], S1, 0, 0, 0);
        else
          S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[j >> 1], S0, 0, 0, 0);
      }
      // keep this order: the scheduler would otherwise sink each read next to
      // its MFMA and the matrix core would wait out the LDS latency every time
      __builtin_amdgcn_sched_barrier(0);
    }
    p_vis = false;
    s_vis = false;
    if (k >= cnt) return;
    const int t = tile_of(k);
    if (t != cur_tile) {
      // group A moving from t0 to t1 (Q of t1 staged in LDS): the scores above
      // used t0's Q; finish t0, then redo S with t1's Q.
      store_tile(cur_tile);
      reset_state();
      load_q_lds();
      cur_tile = t;
      S0 = f32x16{};
      S1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kbase, kr0, sw0, ks), qreg[ks], S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kbase, kr1, sw1, ks), qreg[ks], S1, 0, 0, 0);
      }
    }
    const int q0 = t * kBM + wg * 32;
    const int kv0 = kv_of(k) * kBN;
    s_vis = kv0 < Skv && (!causal || kv0 <= q0 + 31 + off);
    s_kv0 = kv0;
    s_q0 = q0;
  };

  // Vector slot: softmax of the block in S0/S1 -> P, with the online update.
  // The exponent reference m_run only has to keep the probabilities in range,
  // not to be the exact row maximum (any reference gives the same normalised
  // result). So a block is first exponentiated against the current reference
  // without looking for its maximum; only when a row has no reference yet, or
  // when a row's partial sum shows that the block rose far above it
  // (> 2^16), is the block's maximum taken, the reference raised (lazily, by
  // more than kTau) with O and l rescaled, and the block redone.
  // The slot first issues the loads of V of block k into sVc (free since the
  // PV of block k-2), so the MFMA slot carries only the K loads: the direct-
  // to-LDS issue (address and M0 set-up, and for the cache variant the page
  // lookup) then overlaps the exponentials instead of delaying the MFMAs.
  auto vslot = [&](int k, __bf16* sVc) __attribute__((always_inline)) {
    {
      const long prv = page_row(kv_of(k), k < cnt);
#pragma unroll
      for (int n = 0; n < C::NI; ++n) dma_one(vbh, sVc, voff, kv_of(k), k < cnt, n, prv);
    }
    if (!s_vis) return;
    const int kv0 = s_kv0, q0 = s_q0;
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
    float alpha = 1.f;
    auto raise_to_max = [&]() __attribute__((always_inline)) {
      float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[r], S1[r]));
      mx = pair_max(mx);
      const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
      if (cand > m_run + kTau) {
        alpha *= fast_exp2(m_run - cand);
        m_run = cand;
      }
    };
    float la, lb;
    // Masked scores are -inf: with c > 0 and mu finite their exp2 is exactly 0.
    // The row sum adds the fp32 probabilities with plain adds (a dot-product
    // instruction would wait for the matrix core, which the other wave on the
    // SIMD keeps busy); PV uses the same values rounded to bf16.
    auto exponentiate = [&]() __attribute__((always_inline)) {
      const float mu = (m_run == -INFINITY) ? 0.f : m_run;
      la = 0.f;
      lb = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(sub ? S1[r] : S0[r], c, -mu));
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint4 w;
          w.x = pack_bf16x2(e[8 * s + 0], e[8 * s + 1]);
          w.y = pack_bf16x2(e[8 * s + 2], e[8 * s + 3]);
          w.z = pack_bf16x2(e[8 * s + 4], e[8 * s + 5]);
          w.w = pack_bf16x2(e[8 * s + 6], e[8 * s + 7]);
          P[sub][s] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
          for (int r = 0; r < 8; r += 2) {
            la += e[8 * s + r];
            lb += e[8 * s + r + 1];
          }
        }
      }
    };
    const bool exact = __any(m_run == -INFINITY);
    if (exact) raise_to_max();
    exponentiate();
    // !(x <= bound) also catches an infinite or NaN sum
    if (!exact && __any(!(la + lb <= kRedo))) {
      raise_to_max();
      exponentiate();
    }
    l_run = alpha * l_run + (la + lb);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    p_vis = true;
  };

  // ---- prologue: zero this group's V slot of stage 1 (the first MFMA slot
  // reads it with zero probabilities), first K block and first Q tile of each
  // group; group B shares its Q tile (group A's second) through LDS.
  {
    uint4* z = (uint4*)(sV1 + grp * C::ELEMS) + wg * (C::ELEMS / 8 / 4);
#pragma unroll
    for (int i = 0; i < C::ELEMS / 8 / 4 / 64; ++i) z[i * 64 + lane] = make_uint4(0, 0, 0, 0);
  }
  if (CACHE && grp == 0 && nA0 == 0 && t0 != t1) {
    // tile t0 sees no key at all (causal, Skv < Sq): its rows are zeros
    reset_state();
    store_tile(t0);
  }
  if (cnt > 0) {
    dma(kbh, sK0, koff, kv_of(0));
    cur_tile = tile_of(0);
    reset_state();
    load_q_global(cur_tile);
  }
  if (grp == 1 && cntA > nA0 && nA0 > 0) share_q();

  // ---- slots. Every wave runs the same sequence M(0) V(0) M(1) V(1) ...,
  // one barrier per slot; group B takes one empty slot first, so its MFMA slots
  // line up with group A's vector slots. Unrolled by 2 blocks so that every LDS
  // stage is a compile-time choice (stage of block k = k & 1). Both groups then
  // pad to the same number of barriers.
  int nbar = 0;
  if (grp == 1) {
    lds_barrier();
    ++nbar;
  }
  // The wave in its MFMA slot gets the higher issue priority, so that its
  // MFMAs and LDS reads go out as soon as they are ready and the softmax wave
  // on the same SIMD fills the remaining issue cycles.
  for (int k = 0; k <= cnt; k += 2) {
    wait_dma();
    lds_barrier();
    __builtin_amdgcn_s_setprio(1);
    mslot(k, sK0, sV1, sK1);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
    if (k < cnt) vslot(k, sV0);
    wait_dma();
    lds_barrier();
    __builtin_amdgcn_s_setprio(1);
    if (k + 1 <= cnt) mslot(k + 1, sK1, sV0, sK0);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
    if (k + 1 < cnt) vslot(k + 1, sV1);
    nbar += 4;
  }
  {
    const int nbA = 4 * (cntA / 2 + 1), nbB = 1 + 4 * (cntB / 2 + 1);
    const int total = max(nbA, nbB);
    for (; nbar < total; ++nbar) lds_barrier();
  }

  // ---- epilogue: group A hands its partial of t1 to group B through LDS.
  wait_dma();
  __syncthreads();
  float* xo = (float*)((wg < 2 ? (char*)sK0 : (char*)sV0)) + (wg & 1) * C::XO;
  float* xml = (float*)sK1 + wg * 128;
  if (grp == 0) {
    if (split) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = O[db][r];
      xml[lane * 2 + 0] = m_run;
      xml[lane * 2 + 1] = l_run;
    } else if (cur_tile >= 0) {
      store_tile(cur_tile);
    }
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
  const bool cache = p.lens != nullptr;
  // cache: one work-group per (tile, head, sequence), padded to whole rounds of
  // (sequence, kv head) groups per XCD (the padding work-groups exit at once)
  const long groups = (long)p.B * p.Hkv, per_group = (long)(p.Hq / p.Hkv) * p.nT;
  dim3 grid(cache ? (unsigned)(kXcds * ((groups + kXcds - 1) / kXcds) * per_group) : (unsigned)(p.nP * p.Hq * p.B));
  dim3 block(512);
  if (d == 128 && !cache)
    return launch_kernel(prefill_bf16_kernel<128, false>, grid, block, stream, p);
  else if (d == 96 && !cache)
    return launch_kernel(prefill_bf16_kernel<96, false>, grid, block, stream, p);
  else if (d == 64 && !cache)
    return launch_kernel(prefill_bf16_kernel<64, false>, grid, block, stream, p);
  else if (d == 128)
    return launch_kernel(prefill_bf16_kernel<128, true>, grid, block, stream, p);
  else if (d == 96)
    return launch_kernel(prefill_bf16_kernel<96, true>, grid, block, stream, p);
  else if (d == 64)
    return launch_kernel(prefill_bf16_kernel<64, true>, grid, block, stream, p);
  else
    return hipErrorInvalidValue;
}

}  // namespace fa
