// fa_api.hip - the extern "C" entry points declared in include/fa.h.
// Validates every argument on the host (no device access, no allocation, no
// synchronisation), then enqueues the gfx950 kernels on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int kMinDefaultTps = 64;
constexpr int kMaxDefaultTps = 1024;
constexpr int kTargetSplitGroups = 512;  // two resident split work-groups per CU
constexpr int kDefaultSplitGroups = 256; // default split size: grid near one work-group per CU
constexpr int kMaxTps = 2048;
constexpr int kOneLaunchMaxLen = 512;  // default: one split per sequence up to this capacity
constexpr int kCompactMaxB = 4096;  // up to 16 sequences scanned per thread of a split work-group
constexpr int kMaxGridYZ = 65535;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

fa_status check_prefill(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq,
                        int Skv, int d, float scale, int causal) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || d <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (B > kMaxGridYZ || Hq > kMaxGridYZ) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (causal && Sq > Skv) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  // the bf16 kernels run one work-group per (pair of 128-row query tiles, or
  // one tile for the other head dims, head, batch)
  const long tiles = ((long)Sq + 31) / 32;  // (the key-split kernel's tiles: 32 rows at d = 32)
  if (tiles * Hq * B > (long)INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

fa::PrefillParams make_prefill(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                               int Sq, int Skv, float scale, int causal) {
  fa::PrefillParams p;
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv;
  // c = |scale| * log2(e), kept >= 1e-30: with scale = 0 every score scales to
  // ~0 (uniform weights, as the definition gives) while a masked score of -inf
  // still scales to -inf, so exp2 returns exactly 0 for it.
  p.c = fmaxf(fabsf(scale) * fa::kLog2e, 1e-30f);
  p.neg = scale < 0.f ? 1 : 0;
  p.causal = causal;
  p.nT = (Sq + 127) / 128;
  p.nP = (p.nT + 1) / 2;
  return p;
}

// Split work-groups resident at once on the current device: two per compute
// unit (the split kernel's registers and LDS allow two). Cached per device.
int resident_split_groups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kTargetSplitGroups;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return kTargetSplitGroups;
  v = 2 * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Work-groups one split of every sequence launches: B * Hkv * ceil(G / 16).
long split_streams(int B, int Hq, int Hkv) { return (long)B * Hkv * ((Hq / Hkv + 15) / 16); }

// tokens_per_split == 0: one split per sequence (a single launch: the split
// kernel writes o and no merge runs) when the capacity is at most
// kOneLaunchMaxLen tokens, or at most kMaxTps with at least max_kv_len / 8
// split streams; else the smallest power of two >= 64 that keeps the grid
// near kDefaultSplitGroups work-groups, capped at 1024 (a 256k-token sequence
// then still has 256 splits). Measured (caches evicted, d = 128, full
// lengths): a split work-group reads ~50 GB/s, so one launch wins once the
// streams together, not one work-group's rate, set the time, or once the
// merge kernel (several us per call) costs more than a short capacity saves
// by splitting (max_kv_len 512: one launch at every batch; 1024 from 128
// streams; 2048 from 256 streams, e.g. 57.6 against 65.7 us at B = 32,
// Hkv = 8); and fewer, longer splits (about one work-group per CU) beat
// twice as many half as long (B = 4, max_kv_len 2048: 19.3 against 20.7 us).
// Any other value is taken as given (validated by the caller). Returns 0
// for invalid sizes.
int resolve_tps(int B, int Hq, int Hkv, int max_kv_len, int tps) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_kv_len <= 0 || Hq % Hkv != 0) return 0;
  if (tps != 0) return tps;
  const long streams = split_streams(B, Hq, Hkv);
  if (max_kv_len <= kOneLaunchMaxLen || (max_kv_len <= kMaxTps && 8 * streams >= max_kv_len))
    return (max_kv_len + 31) / 32 * 32;
  const long want = ((long)max_kv_len * streams + kDefaultSplitGroups - 1) / kDefaultSplitGroups;
  int t = kMinDefaultTps;
  while (t < kMaxDefaultTps && t < want) t *= 2;
  return t;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes (<= 0, Hq % Hkv != 0, causal with Sq > Skv, or too large)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head_dim or page_size not provided (d = 32, 64, 96, 128, 256; page_size 16)";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointers must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a launch";
    case FA_ERR_ARG: return "FA_ERR_ARG: invalid argument (scale not finite, causal not 0/1, bad tokens_per_split)";
  }
  return "FA_ERR_UNKNOWN";
}

int fa_version(void) { return 200; }

fa_status fa_prefill(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq, int Skv,
                     int d, float scale, int causal, void* stream) {
  fa_status st = check_prefill(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, scale, causal);
  if (st != FA_OK) return st;
  fa::PrefillParams p = make_prefill(q, k, v, o, B, Hq, Hkv, Sq, Skv, scale, causal);
  if (d == 64 || d == 96 || d == 128) return from_hip(fa::launch_prefill_bf16(p, d, (hipStream_t)stream));
  p.cus = resident_split_groups() / 2;
  return from_hip(fa::launch_prefill_hd(p, d, (hipStream_t)stream));
}

fa_status fa_prefill_cache(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                           const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int Sq, int d, int max_kv_len,
                           int page_size, float scale, int causal, void* stream) {
  if (!seqlens) return FA_ERR_NULL;
  // the checks of fa_prefill with Skv = max_kv_len, without its causal bound
  // Sq <= Skv (here a row with no visible key gives zeros)
  fa_status st = check_prefill(q, kcache, vcache, o, B, Hq, Hkv, Sq, max_kv_len, d, scale, 0);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (block_table && page_size != 16) return FA_ERR_UNSUPPORTED;
  if (!aligned4(seqlens) || (block_table && !aligned4(block_table))) return FA_ERR_ALIGN;
  if (!block_table && (size_t)B * (size_t)max_kv_len > (size_t)INT32_MAX) return FA_ERR_SHAPE;
  // one work-group per (query tile, head, sequence), padded to whole rounds of
  // (sequence, kv head) groups on the 8 XCDs (tiles of 32 rows at the least)
  const long tiles = ((long)Sq + 31) / 32;
  if (8 * (((long)B * Hkv + 7) / 8) * (Hq / Hkv) * tiles > (long)INT32_MAX) return FA_ERR_SHAPE;
  fa::PrefillParams p = make_prefill(q, kcache, vcache, o, B, Hq, Hkv, Sq, max_kv_len, scale, causal);
  p.lens = seqlens;
  p.bt = block_table;
  p.max_len = max_kv_len;
  p.pps = (max_kv_len + 15) / 16;
  if (d == 64 || d == 96 || d == 128) return from_hip(fa::launch_prefill_bf16(p, d, (hipStream_t)stream));
  p.cus = resident_split_groups() / 2;
  return from_hip(fa::launch_prefill_hd(p, d, (hipStream_t)stream));
}

fa_status fa_prefill_f32(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq,
                         int Skv, int d, float scale, int causal, void* stream) {
  fa_status st = check_prefill(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, scale, causal);
  if (st != FA_OK) return st;
  fa::PrefillParams p = make_prefill(q, k, v, o, B, Hq, Hkv, Sq, Skv, scale, causal);
  return from_hip(fa::launch_prefill_f32(p, d, (hipStream_t)stream));
}

int fa_decode_split_tokens(int B, int Hq, int Hkv, int max_kv_len, int tokens_per_split) {
  const int tps = resolve_tps(B, Hq, Hkv, max_kv_len, tokens_per_split);
  if (tps <= 0 || tps % 32 != 0 || tps > kMaxTps) return 0;
  return tps;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_kv_len, int tokens_per_split) {
  const int tps = fa_decode_split_tokens(B, Hq, Hkv, max_kv_len, tokens_per_split);
  if (d <= 0 || tps <= 0) return 0;
  const size_t nsplit = ((size_t)max_kv_len + tps - 1) / tps;
  const size_t rows = (size_t)B * Hq * nsplit;
  return round_up(rows * d * sizeof(float), 256) + round_up(rows * sizeof(float), 256) + 256;
}

}  // extern "C"

namespace {

// Device scratch of fa_decode_noalloc: the split partials, their lse and the
// split-size word of one call, in place of a caller's workspace. Each GPU the
// library runs on holds its own copy for the life of the process. Host code
// never uses the array's name as an address (on the host it is only a stand-in
// for the symbol): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept below.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device); nullptr and the runtime's status if it cannot be found.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !p) return nullptr;
  scratch_addr[dev].store(p, std::memory_order_release);
  return p;
}

// fa_decode, fa_decode_fp8 and fa_decode_int8: the same checks and plan; the
// one-byte caches carry a positive finite scale per tensor.
fa_status decode_common(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                        const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                        int tokens_per_split, float scale, int fmt, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, void* stream, bool use_scratch = false) {
  if (!q || !kcache || !vcache || !seqlens || !o) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_kv_len <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (block_table && page_size != 16) return FA_ERR_UNSUPPORTED;
  const int tps = fa_decode_split_tokens(B, Hq, Hkv, max_kv_len, tokens_per_split);
  if (tps <= 0) return FA_ERR_ARG;
  if (!isfinite(scale)) return FA_ERR_ARG;
  const bool bytes = fmt != fa::kCacheBf16;
  if (bytes && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o)) return FA_ERR_ALIGN;
  if (!aligned4(seqlens) || (block_table && !aligned4(block_table))) return FA_ERR_ALIGN;
  const int G = Hq / Hkv;
  const int hchunks = (G + 15) / 16;
  const long nsplit_l = ((long)max_kv_len + tps - 1) / tps;
  if (((long)B * nsplit_l + 7) / 8 * 8 * Hkv * hchunks > (long)INT32_MAX) return FA_ERR_SHAPE;
  if (!block_table && (size_t)B * (size_t)max_kv_len > (size_t)INT32_MAX) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, Hq, Hkv, d, max_kv_len, tps);
  if (use_scratch) {
    // the allocation-free variant: the device scratch array, within its size
    if (need > kScratchBytes) return FA_ERR_WORKSPACE;
    hipError_t e;
    workspace = scratch_ptr(&e);
    if (!workspace) return FA_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;

  fa::DecodeParams p;
  p.q = q; p.kc = kcache; p.vc = vcache; p.bt = block_table; p.lens = seqlens; p.o = o;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.max_len = max_kv_len;
  p.pages_per_seq = (max_kv_len + 15) / 16;
  p.tps = tps;
  p.nsplit = (max_kv_len + tps - 1) / tps;
  p.G = G;
  p.hchunks = hchunks;
  // One split per sequence: the split kernel writes o itself and the merge
  // launch is skipped (one kernel per call). Every (sequence, head chunk) then
  // has its work-group, so an empty sequence's rows are written as zeros.
  p.direct = p.nsplit == 1 ? 1 : 0;
  // (d = 256: one split work-group per CU, its registers and LDS allow no second)
  p.cap = d == 256 ? resident_split_groups() / 2 : resident_split_groups();
  // One sequence whose splits all fit one round of resident work-groups, or
  // whose split size is given: the device-side choice of the split size would
  // keep tps (one round at tps is the least), so the scan over seqlens has
  // nothing to do. Its splits are numbered in order instead, and a work-group
  // knows its split (and its block-table entries) before it reads the length.
  const bool one_plain = B == 1 && (tokens_per_split != 0 || (long)Hkv * hchunks * p.nsplit <= p.cap);
  p.compact = (B <= kCompactMaxB && !p.direct && !one_plain) ? 1 : 0;
  p.adapt = (tokens_per_split == 0 && p.compact) ? 1 : 0;
  // the work-groups of neighbouring kv heads on one XCD where their row slices
  // are 32 or 64 bytes (so 4 or 2 of them share every 128-byte line); with
  // 96-byte slices (d = 96, one-byte cache) the split order measured faster
  const int slice = d * (bytes ? 1 : 2);
  p.xcd_group = (slice < 128 && 128 % slice == 0) ? 1 : 0;
  // as in prefill: c > 0 even for scale = 0, so a masked score's exp2 is 0;
  // a one-byte cache's K scale multiplies every score, so it joins c
  p.c = fmaxf(fabsf(scale) * (bytes ? k_scale : 1.0f) * fa::kLog2e, 1e-30f);
  p.vs = bytes ? v_scale : 1.0f;
  p.neg = scale < 0.f ? 1 : 0;
  const size_t rows = (size_t)B * Hq * p.nsplit;
  p.ws_o = (float*)workspace;
  p.ws_lse = (float*)((char*)workspace + round_up(rows * d * sizeof(float), 256));
  p.ws_t = (int*)((char*)p.ws_lse + round_up(rows * sizeof(float), 256));
  return from_hip(fa::launch_decode(p, d, fmt, (hipStream_t)stream));
}

}  // namespace

extern "C" {

fa_status fa_decode(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                    const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                    int tokens_per_split, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(q, kcache, vcache, block_table, seqlens, o, B, Hq, Hkv, d, max_kv_len, page_size,
                       tokens_per_split, scale, fa::kCacheBf16, 1.0f, 1.0f, workspace, workspace_bytes, stream);
}

fa_status fa_decode_fp8(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                        const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                        int tokens_per_split, float scale, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode_common(q, kcache, vcache, block_table, seqlens, o, B, Hq, Hkv, d, max_kv_len, page_size,
                       tokens_per_split, scale, fa::kCacheFp8, k_scale, v_scale, workspace, workspace_bytes, stream);
}

fa_status fa_decode_int8(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                         const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                         int tokens_per_split, float scale, float k_scale, float v_scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_common(q, kcache, vcache, block_table, seqlens, o, B, Hq, Hkv, d, max_kv_len, page_size,
                       tokens_per_split, scale, fa::kCacheInt8, k_scale, v_scale, workspace, workspace_bytes, stream);
}

fa_status fa_merge_lse(const float* o_parts, const float* lse, void* o, float* lse_out, int R, int S, int d,
                       int out_bf16, void* stream) {
  if (!o_parts || !lse || !o) return FA_ERR_NULL;
  if (R <= 0 || S <= 0 || d <= 0) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (!aligned16(o_parts) || !aligned16(o) || !aligned4(lse) || (lse_out && !aligned4(lse_out)))
    return FA_ERR_ALIGN;
  fa::MergeParams m;
  m.o_parts = o_parts; m.lse = lse; m.o = o; m.lse_out = lse_out; m.lens = nullptr; m.tps_dev = nullptr;
  m.R = R; m.S = S; m.Hq = 1; m.tps = 1; m.max_len = 0; m.out_bf16 = out_bf16 ? 1 : 0;
  return from_hip(fa::launch_merge(m, d, (hipStream_t)stream));
}

fa_status fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                            const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int d, int max_kv_len,
                            int page_size, int tokens_per_split, float scale, void* stream) {
  return decode_common(q, kcache, vcache, block_table, seqlens, o, B, Hq, Hkv, d, max_kv_len, page_size,
                       tokens_per_split, scale, fa::kCacheBf16, 1.0f, 1.0f, nullptr, 0, stream, true);
}

}  // extern "C"
