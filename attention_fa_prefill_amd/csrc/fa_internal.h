// fa_internal.h - types and launchers shared by the gfx950 kernels and the
// C-ABI layer. Nothing here is part of the public interface (include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// log2(e): the kernels evaluate exp(x) as exp2(x * log2(e)) with the factor
// folded into the softmax scale.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Enqueues kernel k (which takes one parameter block by value) and returns the
// status of this launch alone. The runtime's pending "last error" is neither
// read nor cleared, so an error the caller left behind is not reported as a
// failure of this call, and stays the caller's to collect.
template <typename P>
inline hipError_t launch_kernel(void (*k)(P), dim3 grid, dim3 block, hipStream_t stream, const P& p) {
  void* args[] = {const_cast<P*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, 0, stream);
}

// ---------------------------------------------------------------- prefill
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, Hq, Hkv, Sq, Skv;
  float c;     // |scale| * log2(e)
  int neg;     // scale < 0: q is negated on load (exact) so that c >= 0
  int causal;  // bottom-right aligned
  int nT;      // query tiles of 128 rows
  int nP;      // work-groups per (b, h): pairs of query tiles
  // KV-cache prefill (bf16 kernel only): lens != nullptr selects it. k, v are
  // then the K / V caches in the decode layouts, Skv = clamp(lens[b], 0, max_len).
  const int32_t* lens = nullptr;
  const int32_t* bt = nullptr;  // block table [B, pps] or nullptr (contiguous cache)
  int max_len = 0, pps = 0;
  int cus = 0;  // compute units of the device (head dim 256 picks its kernel by grid size)
};

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_prefill_hd(const PrefillParams& p, int d, hipStream_t stream);

// ---------------------------------------------------------------- decode
struct DecodeParams {
  const void* q;       // bf16 [B, Hq, d]
  const void* kc;      // bf16 (or FP8 E4M3) rows of [*, Hkv, d]
  const void* vc;
  const int32_t* bt;   // block table or nullptr
  const int32_t* lens; // [B]
  void* o;             // bf16 [B, Hq, d]
  float* ws_o;         // fp32 [B, Hq, nsplit, d]
  float* ws_lse;       // fp32 [B, Hq, nsplit]
  int B, Hq, Hkv, max_len, pages_per_seq, tps, nsplit;
  int G;               // query heads per kv head
  int hchunks;         // ceil(G / 16)
  float c;             // |scale| * log2(e) (one-byte cache: times the K scale)
  float vs;            // V scale (one-byte cache), 1 for bf16
  int neg;
  int compact;         // number live splits densely (B small enough to scan per work-group)
  int adapt;           // compact and default split size: the kernel may enlarge tps
  int cap;             // split work-groups resident at once on this GPU
  int* ws_t;           // the split size the split kernel used (written by work-group 0)
  int direct;          // one split per sequence (nsplit = 1): the split kernel writes o, no merge
  int xcd_group;       // all (kv head, head chunk) work-groups of a split on one XCD (row slices < 128 B)
};

// KV-cache element formats: bf16; one byte per element, OCP FP8 E4M3 codes or
// signed 8-bit integers (K = c-folded scale * code, V = vs * code)
constexpr int kCacheBf16 = 0, kCacheFp8 = 1, kCacheInt8 = 2;
hipError_t launch_decode(const DecodeParams& p, int d, int fmt, hipStream_t stream);

struct MergeParams {
  const float* o_parts;  // [R, S, d]
  const float* lse;      // [R, S] natural log
  void* o;               // [R, d] bf16 or fp32
  float* lse_out;        // [R] or nullptr
  const int32_t* lens;   // if not null: valid splits of row r = ceil(clamp(lens[r / Hq]) / split size)
  const int* tps_dev;    // if not null: the split size, in device memory (else tps)
  int R, S, Hq, tps, max_len, out_bf16;
};

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t stream);

}  // namespace fa
