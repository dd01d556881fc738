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
// up to 16 query heads sharing g, split s of T tokens), live splits numbered
// densely so that the XCDs get equal shares of a mixed-length batch (a single
// sequence whose splits fit one round is numbered in order, and its
// work-groups read their block-table entries beside its length). T is the
// caller's split size, or with the default one of a few sizes chosen from
// seqlens on the device, so that the live splits fill whole rounds of
// resident work-groups. Waves take 32-token
// steps round-robin and keep two steps of loads in flight. Per step:
//   - K rows go HBM -> VGPRs directly in the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (16 tokens x 32 dims per MFMA);
//   - V rows go HBM -> the wave's LDS stage with direct-to-LDS buffer loads
//     (16 bytes per lane, swizzled), and come back through ds_read_b64_tr_b16
//     as the A operand of O^T += V^T . P^T;
//   - S^T = K . Q^T for all query heads of the group at once (Q^T lives in
//     VGPRs; unused head columns are zero), so the FLOPs ride on MFMA and the
//     vector ALU only runs the softmax;
//   - online softmax per head with a lazily raised running max.
// Every load goes through a buffer resource whose record count ends at the
// last valid token row of its page, so rows past the sequence length (and the
// slack of the last page) read as zero without touching memory; their scores
// are set to -inf. Block-table entries past the last page are never used.
// At the end the 4 waves' states are merged in LDS and the split writes its
// normalised output and natural-log log-sum-exp to the workspace.
//
// Paged and contiguous caches run the same instructions in the same order and
// differ only in the row address, so their results are bitwise equal.
//
// An FP8 E4M3 cache (one byte per element, one scale per tensor) runs the same
// kernel: K is widened to bf16 in registers, V goes to LDS as bytes and comes
// back through the 8-bit transpose read, both exactly; the K scale is folded
// into the softmax factor and the V scale into each split's output.
//
// Merge kernel: per row, M = max lse_s, w_s = exp(lse_s - M),
// o = sum_s w_s o_s / sum_s w_s, lse = M + log(sum_s w_s); empty splits skipped.
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kStep = 32;      // tokens per wave step
constexpr float kTau = 8.0f;   // lazy rescale threshold (log2 units)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// V staging swizzle: 16-byte chunk XOR 2*(row % 8) with 16 or more chunks per
// LDS row, 2*(row % (CP/2)) with fewer, so the 4-row x 32-byte footprint of
// each transpose read hits distinct banks. (CP: 16-byte chunks per LDS row of
// the stage, a power of two; rows of d = 96 are padded to it.)
template <int CP>
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & (CP >= 16 ? 7 : CP / 2 - 1)); }
// FP8 V staging swizzle. A transpose read of 8-bit elements (ds_read_b64_tr_b8)
// by 16 lanes covers one 16-byte chunk of 8 rows: tokens 4cq..4cq+3 and
// 16+4cq..16+4cq+3 of the step. XOR with a function of the row that differs
// on those 8 rows (8 or 16 chunks per row) or, with the row's parity, still
// separates them (4 chunks per 64-byte row) places the 8 reads in distinct
// banks.
template <int CP>
__device__ __forceinline__ int swz_v8(int row) {
  return CP >= 8 ? ((row & 3) | (((row >> 4) & 1) << 2)) : (((row >> 1) & 1) | (((row >> 4) & 1) << 1));
}

constexpr int pow2_at_least(int x, int lo) {
  int r = lo;
  while (r < x) r *= 2;
  return r;
}
constexpr uint32_t kPadOffset = 0x80000000u;  // a buffer offset past any page: the load returns zeros

// Waits for this wave's vector-memory loads (direct-to-LDS included) until at
// most N are outstanding. The memory clobber keeps LDS reads of a stage from
// being scheduled above the wait that covers that stage's loads.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kMaxTps = 2048;            // tokens per split at most
constexpr int kMaxPages = kMaxTps / 16;  // pages per split
constexpr int kCand = 4;                 // default split sizes tried: tps * {4, 5, 6, 8} / 4
__host__ __device__ constexpr int cand_quarters(int u) { return u == 3 ? 8 : 4 + u; }
constexpr int kPageSlots = kMaxPages + 32;  // + the pages of the loads issued past the end

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// 8 OCP FP8 E4M3 codes (byte i of x = element i) -> 8 bf16, exactly (every
// E4M3 value is a bf16 value); the per-tensor scale is applied elsewhere.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 x) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 signed 8-bit integers in two's complement (byte i of x = element i) -> 8
// bf16, exactly (every integer in -128..127 is a bf16 value); the per-tensor
// scale is applied elsewhere.
__device__ __forceinline__ bf16x8 int8x8_to_bf16(u32x2 x) {
  auto e = [](uint32_t w, int k) __attribute__((always_inline)) { return (float)((int)(w << (24 - 8 * k)) >> 24); };
  const uint4 r = make_uint4(pack2(e(x.x, 0), e(x.x, 1)), pack2(e(x.x, 2), e(x.x, 3)),
                             pack2(e(x.y, 0), e(x.y, 1)), pack2(e(x.y, 2), e(x.y, 3)));
  return __builtin_bit_cast(bf16x8, r);
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP: shifts by 1, 2,
// 4 and 8 lanes inside each row of 16 (lanes shifted in from outside the row
// add 0), then the last lane of row 0 (of row 2) is added to row 1 (to row 3)
// and the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// F8: the cache holds one byte per element, OCP FP8 E4M3 codes (I8 false) or
// signed 8-bit integers (I8 true), with one scale per tensor: K = p.ks * code,
// V = p.vs * code. p.ks is folded into the softmax factor c by the host and
// p.vs is applied to each split's output; K and V are widened to bf16
// exactly, so the arithmetic is that of the bf16 cache on the dequantised
// values.
// Waves per SIMD the split kernel is compiled for: one-byte caches at d <= 128
// keep their registers and LDS within three work-groups per CU (a step there
// moves half the bytes for the same per-token work, so more waves keep more
// bytes in flight); bf16 two; d = 256 one.
template <int D, bool F8>
constexpr int split_waves_per_simd() { return D > 128 ? 1 : (F8 ? 3 : 2); }

template <int D, bool F8, bool I8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(split_waves_per_simd<D, F8>())))
decode_split_kernel(DecodeParams p) {
  static_assert(F8 || !I8, "the int8 cache is a one-byte cache");
  auto byte8_to_bf16 = [](u32x2 x) __attribute__((always_inline)) {
    if constexpr (I8)
      return int8x8_to_bf16(x);
    else
      return fp8x8_to_bf16(x);
  };
  constexpr int ES = F8 ? 1 : 2;     // bytes per cached element
  constexpr int KS = D / 32;         // k-steps of S^T = K . Q^T (16x16x32)
  constexpr int DB = D / 16;         // 16-dim blocks of O^T
  constexpr int CH = D * ES / 16;    // 16-byte chunks per row
  // LDS stage rows hold CP chunks, a power of two (so the XOR swizzles stay
  // inside the row) and at least 4 (so a direct-to-LDS load stays inside one
  // page of 16 rows): d = 96 rows and d = 32 FP8 rows are padded; the lanes
  // that land on padding chunks load nothing and write zeros.
  constexpr int CP = pow2_at_least(CH, 4);
  constexpr int RB = CP * 16;        // bytes per LDS stage row
  constexpr int RI = 64 / CP;        // V rows per direct-to-LDS load (bf16 D=128: 4; fp8: 8)
  constexpr int VDMA = kStep / RI;   // direct-to-LDS loads per step
  constexpr int NLD = 2 * KS + VDMA; // vector-memory instructions issued per step
  // Two V stages per wave (the step being used and the one in flight), kStep
  // rows of RB bytes each (sized in bf16 units). Together they also hold the
  // exchange of the 4 waves' states at the end: 32-dim-block halves of O^T,
  // blocks [0, HD) in the first stage and [HD, DB) in the second.
  constexpr int STG = kStep * RB / 2;
  constexpr int HD = (DB + 1) / 2;
  static_assert(HD * 4 * 64 * 4 <= STG * 2, "a stage holds half of a wave's O^T");
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[4][STG];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[4][STG];
  __shared__ float sM[4][64], sL[4][64];
  __shared__ int sRow0[kPageSlots];  // first cache row of each page of this split

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work items: (kv head, query-head chunk) pairs gh times split items (the
  // splits of all sequences); the grid is padded to whole groups of 8 split
  // items. Work-group L runs on XCD L % 8.
  //  - p.xcd_group: the work-groups of all gh of one split item go to one XCD,
  //    so those that read the same cache lines meet in one L2. The host sets
  //    it where a kv head's slice of a token row is 32 or 64 bytes (d *
  //    bytes per element), so that 4 or 2 neighbouring kv heads share every
  //    128-byte line: otherwise each line is fetched once per XCD that reads
  //    it (4x or 2x the bytes, measured), and grouped the call is 3-9 %
  //    faster.
  //  - otherwise L = gh * (split items) + item: each gh's splits in a run.
  //    Where no lines, or only some, are shared this order is as fast or up
  //    to 6 % faster (measured at d = 96, 128 and 256, and with head chunks
  //    of one kv head, which read the same rows, on different XCDs).
  const int nGH = p.Hkv * p.hchunks;
  int gh = 0, item = 0;
  auto map_item = [&](int n_items) __attribute__((always_inline)) {
    const int L = blockIdx.x;
    if (p.xcd_group) {
      gh = (L / 8) % nGH;
      item = (L / 8 / nGH) * 8 + L % 8;
      return item < n_items;
    }
    gh = n_items > 0 ? L / n_items : 0;
    item = n_items > 0 ? L % n_items : 0;
    return L < nGH * n_items;
  };
  int T = p.tps;  // tokens per split of this call
  auto splits_of = [&](int l) __attribute__((always_inline)) {
    l = l < 0 ? 0 : (l > p.max_len ? p.max_len : l);
    return (l + T - 1) / T;
  };
  int b, s;
  if (p.compact) {
    // Live splits are numbered densely, sequence by sequence (the same
    // numbering for every gh), so the first work-groups of the grid (the ones
    // the dispatcher starts first) all carry work, every XCD gets an equal
    // share whatever the length mix, and the work-groups past the last live
    // split exit at once.
    // Each thread counts the splits of a run of sequences; a block-wide scan
    // gives the run offsets; the thread whose run holds this item finds it.
    //
    // With the default split size the counts (and scans) are taken for
    // tps * {1, 5/4, 3/2, 2} (multiples of 32, at most kMaxTps) in the same
    // pass, and the size with the fewest tokens per work-group slot over the
    // rounds of resident work-groups its live splits need wins (the smaller on
    // a tie): a batch whose splits overrun one round by a few then runs in one
    // round of slightly longer splits instead of two.
    __shared__ int sWave[4][kCand], sItem[2];
    const int C = (p.B + 255) / 256;
    const int b0 = tid * C, b1 = min(p.B, b0 + C);
    int cand[kCand], cnt[kCand], inc[kCand];
#pragma unroll
    for (int u = 0; u < kCand; ++u) {
      cand[u] = u == 0 ? p.tps : min(kMaxTps, (p.tps * cand_quarters(u) / 4 + kStep - 1) / kStep * kStep);
      cnt[u] = 0;
    }
    for (int bb = b0; bb < b1; ++bb) {
      int l = p.lens[bb];
      l = l < 0 ? 0 : (l > p.max_len ? p.max_len : l);
      cnt[0] += (l + cand[0] - 1) / cand[0];
      if (p.adapt) {
#pragma unroll
        for (int u = 1; u < kCand; ++u) cnt[u] += (l + cand[u] - 1) / cand[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kCand; ++u) {
      inc[u] = (u > 0 && !p.adapt) ? cnt[u] : wave_inclusive_sum(cnt[u]);
      if (lane == 63) sWave[w][u] = inc[u];
    }
    __syncthreads();
    int cs = 0;  // the candidate taken
    if (p.adapt) {
      // uniform values: scalar arithmetic (the grid of any candidate fits in
      // 32 bits: it is at most the grid at tps, which the host checked)
      unsigned long long best = ~0ull;
#pragma unroll
      for (int u = 0; u < kCand; ++u) {
        const unsigned n = (unsigned)(p.Hkv * p.hchunks) *
                           (unsigned)__builtin_amdgcn_readfirstlane(sWave[0][u] + sWave[1][u] + sWave[2][u] + sWave[3][u]);
        const unsigned long long cost = (unsigned long long)((n + p.cap - 1) / (unsigned)p.cap) * (unsigned)cand[u];
        if (cost < best) {
          best = cost;
          cs = u;
        }
      }
    }
    int mycnt = cnt[0], myinc = inc[0];
    T = cand[0];
#pragma unroll
    for (int u = 1; u < kCand; ++u)
      if (u == cs) {
        mycnt = cnt[u];
        myinc = inc[u];
        T = cand[u];
      }
    if (blockIdx.x == 0 && tid == 0) *p.ws_t = T;  // read by the merge
    int before = 0, total = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      before += u < w ? sWave[u][cs] : 0;
      total += sWave[u][cs];
    }
    if (!map_item(total)) return;  // past the last live split (uniform)
    const int excl = before + myinc - mycnt;
    if (item >= excl && item < excl + mycnt) {
      int acc = excl;
      for (int bb = b0; bb < b1; ++bb) {
        const int n = splits_of(p.lens[bb]);
        if (item < acc + n) {
          sItem[0] = bb;
          sItem[1] = item - acc;
          break;
        }
        acc += n;
      }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(sItem[0]);
    s = __builtin_amdgcn_readfirstlane(sItem[1]);
    if (b < 0 || b >= p.B || s < 0 || s >= p.nsplit) return;  // cannot happen: every live item has an owner
  } else {
    if (blockIdx.x == 0 && tid == 0) *p.ws_t = T;  // read by the merge
    if (!map_item(p.B * p.nsplit)) return;  // grid padding (uniform)
    s = item % p.nsplit;
    b = item / p.nsplit;
  }
  const int g = gh / p.hchunks, hc = gh % p.hchunks;
  const int tok0 = s * T;
  // This split's pages of the block table are read before the length, as
  // their addresses do not depend on it (the two reads overlap instead of
  // following each other): thread i reads the page tok0 / 16 + i of the
  // split's at most T / 16, within the row; entries past the sequence's last
  // page are read but not used.
  static_assert(kPageSlots <= 256, "one page slot per thread");
  const int my_pg = tok0 / 16 + tid;
  int my_page = 0;
  if (p.bt && tid * 16 < T && my_pg < p.pages_per_seq) my_page = p.bt[(size_t)b * p.pages_per_seq + my_pg];
  int len = p.lens[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int hq0 = g * p.G + hc * 16;
  const int nh = min(16, p.G - hc * 16);
  if (tok0 >= len) {
    // empty split: the merge never reads it. (direct: the sequence is empty
    // and its rows of o are zeros, the value of an empty sum.)
    if (p.direct) {
      __bf16* o = (__bf16*)p.o + ((size_t)b * p.Hq + hq0) * D;
      for (int i = tid; i < nh * D / 8; i += 256) ((uint4*)o)[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int tok1 = min(len, tok0 + T);
  const int nsteps = (tok1 - tok0 + kStep - 1) / kStep;
  const int Hkv = p.Hkv;

  // Pages past the end of the sequence get row 0: their loads have a zero
  // record count and never touch memory.
  const int npg = (tok1 - tok0 + 15) / 16;
  if (tid < kPageSlots) sRow0[tid] = tid < npg ? (p.bt ? my_page * 16 : b * p.max_len + my_pg * 16) : 0;
  __syncthreads();

  const int n = lane & 15, cq = lane >> 4;  // MFMA column (head / token) and k-group
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

  // Buffer resource over page pi (relative to the split) of kv head g: its
  // record count ends right after the last valid token row, so rows past the
  // sequence length read as zero (K: masked score; V: no NaN can leak).
  const size_t rowstride = (size_t)Hkv * D * ES;  // bytes between consecutive tokens
  auto page_rsrc = [&](const void* cache, int pi) __attribute__((always_inline)) {
    const int nvalid = max(0, min(16, tok1 - (tok0 + 16 * pi)));
    const int row0 = __builtin_amdgcn_readfirstlane(sRow0[pi]);
    const char* base = (const char*)cache + ((size_t)row0 * Hkv + g) * (size_t)(D * ES);
    const int nrec = max(0, (nvalid - 1) * (int)rowstride + D * ES);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, kRsrcWord3);
  };
  // K operand of one 32-token step: half h = page 2st+h, lane (n, cq) holds
  // K[token n of the page][32 ks + 8 cq .. +8] - the A layout of 16x16x32.
  // (FP8: 8 bytes of codes per lane, widened at use.)
  using KReg = typename std::conditional<F8, u32x2, u32x4>::type;
  const int koff = (int)((size_t)n * rowstride) + 8 * ES * cq;
  auto load_k = [&](int st, KReg (&kb)[2][KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.kc, 2 * st + h);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (F8)
          kb[h][ks] = __builtin_amdgcn_raw_buffer_load_b64(rs, koff + 32 * ks, 0, 0);
        else
          kb[h][ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, koff + 64 * ks, 0, 0);
      }
    }
  };
  auto k_operand = [&](const KReg& x) __attribute__((always_inline)) {
    if constexpr (F8)
      return byte8_to_bf16(x);
    else
      return __builtin_bit_cast(bf16x8, x);
  };
  // V rows of one step -> this wave's LDS stage, 16 bytes per lane per load;
  // LDS chunk pc of row r holds logical chunk pc ^ swz(r).
  auto dma_v = [&](int st, __bf16* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int ii = 0; ii < VDMA; ++ii) {
      const int r = ii * RI + lane / CP, pc = lane % CP;
      const int h = (ii * RI) / 16;  // page of this load (uniform)
      const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.vc, 2 * st + h);
      const int sw = F8 ? swz_v8<CP>(r) : swz_v<CP>(r);
      const int lc = pc ^ sw;  // logical chunk of the row
      const int voff = lc < CH ? (int)((size_t)(r & 15) * rowstride) + (lc << 4) : (int)kPadOffset;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + ii * 64 * 8), 16, voff, 0, 0, 0);
    }
  };

  f32x4 O[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;  // FP8: includes the K scale
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int y = lane & 15;
  const int row1 = 4 * cq + (y >> 2), row2 = 16 + 4 * cq + (y >> 2);

  // One 32-token step from K registers kb and V stage `stage`.
  // FP8 V^T operand: lane (cq, j) supplies half j % 2 of chunk db of row
  // t(j / 2), and the transpose read returns to lane j column j of the chunk
  // over those 8 rows, i.e. 8 tokens of dim 16 db + j in the order the score
  // registers hold them.
  const int rho = (lane & 15) >> 1;
  const int trow = rho < 4 ? 4 * cq + rho : 16 + 4 * cq + (rho - 4);
  auto step = [&](int st, const KReg (&kb)[2][KS], const __bf16* stage) __attribute__((always_inline)) {
    const int tb = tok0 + st * kStep;
    f32x4 S[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      S[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) S[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(kb[h][ks]), qop[ks], S[h], 0, 0, 0);
    }
    // S^T lane (n, cq) reg r is token tb + 16 h + 4 cq + r of head n; tokens
    // past the end get -inf (their K rows read as zero).
    if (tb + kStep > tok1) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tb + 16 * h + 4 * cq + r >= tok1) S[h][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                     fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float cand = (mx == -INFINITY) ? -INFINITY : c * mx;
    float alpha = 1.f;
    if (cand > m_run + kTau) {
      alpha = fast_exp2(m_run - cand);
      m_run = cand;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    // masked scores are -inf and c > 0: their exp2 is exactly 0
    uint4 pw;
    pw.x = pack2(fast_exp2(fmaf(S[0][0], c, -mu)), fast_exp2(fmaf(S[0][1], c, -mu)));
    pw.y = pack2(fast_exp2(fmaf(S[0][2], c, -mu)), fast_exp2(fmaf(S[0][3], c, -mu)));
    pw.z = pack2(fast_exp2(fmaf(S[1][0], c, -mu)), fast_exp2(fmaf(S[1][1], c, -mu)));
    pw.w = pack2(fast_exp2(fmaf(S[1][2], c, -mu)), fast_exp2(fmaf(S[1][3], c, -mu)));
    // row sum of the bf16-rounded probabilities (the values PV uses)
    float la = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.x), ones, 0.f, false);
    la = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.y), ones, la, false);
    float lb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.z), ones, 0.f, false);
    lb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.w), ones, lb, false);
    l_run = alpha * l_run + (la + lb);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) O[db] *= alpha;
    }
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
    // O^T += V^T . P^T; contraction index 8 cq + i is token 4 cq + i (i < 4)
    // or 16 + 4 cq + (i - 4) (i >= 4), matching the score registers.
    const char* vslot = (const char*)stage;
    if constexpr (F8) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* a8 = vslot + trow * RB + ((db ^ swz_v8<CP>(trow)) << 4) + 8 * (lane & 1);
        const i32x2 v8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)a8);
        O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(byte8_to_bf16(__builtin_bit_cast(u32x2, v8)), pop, O[db], 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int colb = (16 * db + 4 * (y & 3)) * 2;
      const char* a1 = vslot + row1 * RB + (((colb >> 4) ^ swz_v<CP>(row1)) << 4) + (colb & 15);
      const char* a2 = vslot + row2 * RB + (((colb >> 4) ^ swz_v<CP>(row2)) << 4) + (colb & 15);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a2);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop, O[db], 0, 0, 0);
    }
  };

  // Waves take steps w, w+4, w+8, ...; each wave keeps two steps in flight:
  // K in two register buffers, V in two LDS stages. Every load call issues
  // exactly NLD instructions (those of steps past the end read nothing), so
  // the outstanding-load count at each wait is the same on every path.
  const int nw = nsteps > w ? (nsteps - w + 3) / 4 : 0;
  // kept as raw dwords: a bf16-typed copy across the loop makes the compiler
  // repack the halves, which waits for the loads right after they are issued
  KReg kA[2][KS], kB[2][KS];
  __bf16* stA = sV0[w];
  __bf16* stB = sV1[w];
  // (d = 256: a step is 32 loads, so before a new step's loads go out the
  // pending ones are brought down to 31; the count never exceeds the 63 the
  // wait counter holds)
  constexpr int kRoom = 2 * NLD > 63 ? 63 - NLD : -1;
  dma_v(w, stA);
  load_k(w, kA);
  if constexpr (kRoom >= 0) wait_vm<kRoom>();
  dma_v(w + 4, stB);
  load_k(w + 4, kB);
  for (int i = 0; i < nw; i += 2) {
    wait_vm<NLD>();  // step i's loads are done; step i+1's may be pending
    step(w + 4 * i, kA, stA);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's reads of stage A are done
    if constexpr (kRoom >= 0) wait_vm<kRoom>();
    dma_v(w + 4 * (i + 2), stA);
    load_k(w + 4 * (i + 2), kA);
    wait_vm<NLD>();
    if (i + 1 < nw) step(w + 4 * (i + 1), kB, stB);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if constexpr (kRoom >= 0) wait_vm<kRoom>();
    dma_v(w + 4 * (i + 3), stB);
    load_k(w + 4 * (i + 3), kB);
  }
  wait_vm<0>();  // no direct-to-LDS write may land after the stages are reused

  // ---- merge the 4 waves: O^T lane (n, cq) reg r is dim 16 db + 4 cq + r of head n.
  __syncthreads();
  // exchange slot of 16-dim block db, register r, of wave u's O^T
  auto xslot = [&](int u, int db, int r) __attribute__((always_inline)) {
    return (db < HD ? (float*)sV0[u] : (float*)sV1[u]) + ((db % HD) * 4 + r) * 64 + lane;
  };
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) *xslot(w, db, r) = O[db][r];
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
    __bf16* dst_o = (__bf16*)p.o + ((size_t)b * p.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float acc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) x += a[u] * *xslot(u, db, r);
        acc[r] = x * inv * p.vs;
      }
      // direct (one split per sequence): this split is the whole sequence and
      // its normalised output is o, rounded to bf16 as the merge would round
      // a single split's output (weight exactly 1)
      if (p.direct)
        *(uint2*)(dst_o + 16 * db + 4 * cq) = make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
      else
        *(float4*)(dst + 16 * db + 4 * cq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    if (cq == 0 && !p.direct) p.ws_lse[((size_t)b * p.Hq + hq) * p.nsplit + s] = (M + log2f(L)) * kLn2;
  }
}

// Merge: one work-group of 256 threads per (output row, 32 output dims).
// 8 threads cover a split's 32 dims with one 16-byte load each (one 128-byte
// access per split), 32 split groups stride over the splits, and each thread
// loads 8 splits' log-sum-exps and partial outputs together before using them,
// so a row of up to 256 splits is read in one round trip. Each thread keeps a
// running max and rescales its sums when the max rises (no separate pass for
// the max); the 32 group states are then combined in LDS the same way.
// Splits whose lse is -inf carry no weight and their partial output is ignored.
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(MergeParams p) {
  constexpr int CW = 32;          // output dims per work-group
  constexpr int TPS = CW / 4;     // threads per split
  constexpr int NG = 256 / TPS;   // split groups
  constexpr int U = 8;            // splits per thread per round
  __shared__ float sm[4], sw[NG];
  __shared__ float4 sa[NG][TPS];
  const int tid = threadIdx.x;
  const int r = blockIdx.x, cb = blockIdx.y;
  int nS = p.S;
  if (p.lens) {
    // the split kernel's split size (at least p.tps, so nS <= p.S)
    const int T = p.tps_dev ? min(kMaxTps, max(p.tps, *p.tps_dev)) : p.tps;
    int len = p.lens[r / p.Hq];
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    nS = min(p.S, (len + T - 1) / T);
  }
  const int c = tid % TPS, sg = tid / TPS;
  const float* lse = p.lse + (size_t)r * p.S;
  const float* op = p.o_parts + (size_t)r * p.S * D + CW * cb + 4 * c;
  float m = -INFINITY, W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nS; s0 += NG * U) {
    float l[U];
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NG + sg;
      l[u] = -INFINITY;
      x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < nS) {
        l[u] = lse[s];
        x[u] = *(const float4*)(op + (size_t)s * D);
      }
    }
    float mr = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mr = fmaxf(mr, l[u]);
    if (mr != -INFINITY) {
      const float sc = (m == -INFINITY) ? 0.f : expf(m - mr);
      W *= sc;
      acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (l[u] != -INFINITY) {
          const float wt = expf(l[u] - mr);
          W += wt;
          acc.x = fmaf(wt, x[u].x, acc.x);
          acc.y = fmaf(wt, x[u].y, acc.y);
          acc.z = fmaf(wt, x[u].z, acc.z);
          acc.w = fmaf(wt, x[u].w, acc.w);
        }
      }
      m = mr;
    }
  }
  // combine the groups: M = max of the group maxima, every thread rescales its
  // own group's sums by exp(m - M), then plain sums over the groups
  float M = m;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((tid & 63) == 0) sm[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  const float f = (m == -INFINITY) ? 0.f : expf(m - M);
  acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
  sa[sg][c] = acc;
  if (c == 0) sw[sg] = W * f;
  __syncthreads();
  if (tid < TPS) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
#pragma unroll 8
    for (int g = 0; g < NG; ++g) {
      const float4 xg = sa[g][tid];
      a.x += xg.x; a.y += xg.y; a.z += xg.z; a.w += xg.w;
      wsum += sw[g];
    }
    const bool empty = M == -INFINITY;
    const float inv = empty ? 0.f : 1.0f / wsum;
    const float v0 = a.x * inv, v1 = a.y * inv, v2 = a.z * inv, v3 = a.w * inv;
    const size_t o_off = (size_t)r * D + CW * cb + 4 * tid;
    if (p.out_bf16)
      *(uint2*)((__bf16*)p.o + o_off) = make_uint2(pack2(v0, v1), pack2(v2, v3));
    else
      *(float4*)((float*)p.o + o_off) = make_float4(v0, v1, v2, v3);
    if (p.lse_out && cb == 0 && tid == 0) p.lse_out[r] = empty ? -INFINITY : M + logf(wsum);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, int fmt, hipStream_t stream) {
  // split items padded to a multiple of 8 (one XCD's share of each group of 8)
  dim3 grid(((p.B * p.nsplit + 7) / 8 * 8) * p.Hkv * p.hchunks), block(256);
  hipError_t e;
  if (fmt == kCacheBf16 && d == 128)
    e = launch_kernel(decode_split_kernel<128, false, false>, grid, block, stream, p);
  else if (fmt == kCacheBf16 && d == 64)
    e = launch_kernel(decode_split_kernel<64, false, false>, grid, block, stream, p);
  else if (fmt == kCacheBf16 && d == 256)
    e = launch_kernel(decode_split_kernel<256, false, false>, grid, block, stream, p);
  else if (fmt == kCacheFp8 && d == 128)
    e = launch_kernel(decode_split_kernel<128, true, false>, grid, block, stream, p);
  else if (fmt == kCacheFp8 && d == 64)
    e = launch_kernel(decode_split_kernel<64, true, false>, grid, block, stream, p);
  else if (fmt == kCacheFp8 && d == 256)
    e = launch_kernel(decode_split_kernel<256, true, false>, grid, block, stream, p);
  else if (fmt == kCacheInt8 && d == 128)
    e = launch_kernel(decode_split_kernel<128, true, true>, grid, block, stream, p);
  else if (fmt == kCacheInt8 && d == 64)
    e = launch_kernel(decode_split_kernel<64, true, true>, grid, block, stream, p);
  else if (fmt == kCacheInt8 && d == 256)
    e = launch_kernel(decode_split_kernel<256, true, true>, grid, block, stream, p);
  else if (fmt == kCacheBf16 && d == 96)
    e = launch_kernel(decode_split_kernel<96, false, false>, grid, block, stream, p);
  else if (fmt == kCacheBf16 && d == 32)
    e = launch_kernel(decode_split_kernel<32, false, false>, grid, block, stream, p);
  else if (fmt == kCacheFp8 && d == 96)
    e = launch_kernel(decode_split_kernel<96, true, false>, grid, block, stream, p);
  else if (fmt == kCacheFp8 && d == 32)
    e = launch_kernel(decode_split_kernel<32, true, false>, grid, block, stream, p);
  else if (fmt == kCacheInt8 && d == 96)
    e = launch_kernel(decode_split_kernel<96, true, true>, grid, block, stream, p);
  else if (fmt == kCacheInt8 && d == 32)
    e = launch_kernel(decode_split_kernel<32, true, true>, grid, block, stream, p);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess || p.direct) return e;  // direct: the split kernel wrote o
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
  m.tps_dev = p.ws_t;
  m.max_len = p.max_len;
  m.out_bf16 = 1;
  return launch_merge(m, d, stream);
}

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t stream) {
  dim3 grid(p.R, d / 32), block(256);
  if (d == 128)
    return launch_kernel(merge_kernel<128>, grid, block, stream, p);
  else if (d == 64)
    return launch_kernel(merge_kernel<64>, grid, block, stream, p);
  else if (d == 256)
    return launch_kernel(merge_kernel<256>, grid, block, stream, p);
  else if (d == 96)
    return launch_kernel(merge_kernel<96>, grid, block, stream, p);
  else if (d == 32)
    return launch_kernel(merge_kernel<32>, grid, block, stream, p);
  else
    return hipErrorInvalidValue;
}

}  // namespace fa
