// Paged single-token GQA decode for bf16, head_dim 128, cache blocks of 16,
// 32 or 64 tokens (streamed as 16-token blocks).  The cache
// may hold bf16 or FP8 E4M3FN codes ("Qwen2大模型架构解析与vLLM优化实践",
// §4.1-4.2 FP8 KV-cache quantization with cache scales, §6.3 E4M3FN): FP8
// tiles are half the bytes and are widened to bf16 in registers (exact),
// k_scale folds into the score scale and v_scale into the output.
//
// Attention of one new token over its sequence's paged KV ("vLLM 部署 Qwen",
// §2.1 PagedAttention; §4.1: access to KV pages is what decode tuning is
// about).  GQA: the G = H/Hkv query heads of a group share one KV head
// ("Qwen2 模型结构代码详解", §2), so each (block, KV head) tile is read from HBM
// exactly once and used for all G heads.
//
// Work decomposition.  The work units are the (sequence, KV head, block)
// triples in that order, cut into contiguous ranges.  Persistent 4-wave
// workgroups, two per CU (a wave per SIMD each: while one starts a piece,
// waiting for its first tiles, the other streams), take range i = their
// index first and then claim ranges in order from a device-wide counter.
// The plain decode cuts the units into equal ranges of at least
// kOneTierMin units, two per CU (one per CU for bf16 batches of
// kBf16WideUnits units or more, where the pieces and merges that more
// ranges cut cost more than the overlap wins).  The cascade's private level
// keeps a schedule of shrinking sizes (75% of the units in kCUs ranges, 15%
// in kCUs, 10% in 2 kCUs; one tier from kOneTierUnits), so that CUs and
// XCDs that stream faster (measured: up to ~20% apart) take more of the
// small ranges at the end.  (A first claim by every workgroup at once
// queued ~2.5 us of atomics on the counter before any tile load.)  Which
// ranges a workgroup gets varies; what is computed for each range does not.
// A range covers whole (sequence, KV head) segments, which its workgroup
// finishes itself, and at most two pieces of segments that other ranges
// share: those partial softmax states go to the workspace, and the range
// that completes a shared segment (the last to add its units to the
// segment's arrival counter) combines them exactly, in range order:
//   M = max_r m_r,  L = sum_r l_r 2^(m_r - M),  o = sum_r a_r 2^(m_r - M) / L
// (no separate merge launch: measured, it cost 7-10 us per call).
// Partial states are the only HBM writes besides the output, and while the
// reads saturate HBM every written byte costs several read bytes, so the
// schedule keeps them to about one per range.
// Inside a workgroup the four waves take a piece's blocks round-robin, each
// with its own softmax state, and merge through LDS when the piece ends.
//
// Per block, in a wave:
//   S^T = K q^T with four 16x16x32 bf16 MFMAs: K tile [16][128] (rows
//     256 B); lane (j = lane / 16, r = lane % 16) loads key r, 16-byte pieces
//     at 64 c + 16 j, so every load instruction reads a 64-byte run of each
//     of the 16 keys; q (the B operand, padded to 16 heads with zeros) uses
//     the same dim order.  Lane (j, r) receives head r's scores of keys
//     4j..4j+3.
//   Online softmax per head (column): p = 2^(z scale log2 e - m) rounded to
//     bf16 is already the B operand of P V; the reference m moves only when
//     a block's maximum exceeds it by more than kLazy.
//   O^T += V^T P^T with eight 16x16x16 bf16 MFMAs (one per 16 dims): V tile
//     [128][16] dims major; lane (j, r) loads dim 16 t + r, keys 4j..4j+3, so
//     every load instruction reads 512 contiguous bytes.
// Results depend only on the logical sizes (never on the physical block
// placement) and are bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace qw {

constexpr int kBlk = 16;                // tokens per cache block
constexpr int kD = 128;                 // head_dim
constexpr int kMaxG = 8;
#ifndef QW_DECODE_NBUF
#define QW_DECODE_NBUF 3
#endif
constexpr int kNBuf = QW_DECODE_NBUF;   // blocks (K and V tiles) in flight per wave
constexpr int kNW = 4;                  // waves per workgroup, one per SIMD
constexpr int kThreads = kNW * 64;
constexpr int kCUs = 256;               // workgroups per round of the schedule
constexpr int kTiers = 3;
// The cascade's schedule: tier t takes units [U pct[t] / 100, U pct[t + 1] /
// 100) in equal ranges of at least kTierMin[t] units, at most kTierWgs[t] of
// them (the host sizes the workspace for the bound it knows; the kernels
// count the ranges for the actual U).  Batches of at least kOneTierUnits
// units (128 blocks per CU) take one tier: equal ranges, one per CU, the two
// later tiers empty.  There the shrinking tiers cost more in pieces and
// merges than their balancing wins (measured on the plain decode: the long
// decode 295 -> 284 us, the mixed step's 96 decodes 91 -> 86 us); smaller
// batches keep them (a cascade's 64 short suffixes: 99 against 122 us with
// one tier).
__constant__ int kTierPct[kTiers + 1] = {0, 75, 90, 100};
__constant__ int kOneTierPct[kTiers + 1] = {0, 100, 100, 100};
constexpr int kTierPctHost[kTiers + 1] = {0, 75, 90, 100};
constexpr int64_t kOneTierUnits = 128 * 256;
constexpr int kTierWgs[kTiers] = {kCUs, kCUs, 2 * kCUs};
__constant__ int kTierMin[kTiers] = {64, 32, 24};
constexpr int kTierMinHost[kTiers] = {64, 32, 24};
// The plain decode's schedule (above): equal ranges of at least
// kOneTierMin units, at most kPlainRanges of them (kCUs for a bf16 batch of
// kBf16WideUnits units or more).  Measured per call, two workgroups per CU
// in both, against the cascade's schedule: the Qwen3-0.6B-shaped decode
// (17K units) 42.2 -> 38.1 us, the mixed step's decodes (47K) 81.2 -> 78.2,
// the FP8 long decode (215K) 170.2 -> 166.6; the bf16 long decode (215K)
// 277.0 us with 256 ranges against 282.0 with 512.
constexpr int kOneTierMin = 32;
constexpr int kPlainRanges = 2 * kCUs;
constexpr int64_t kBf16WideUnits = 256 * kCUs;
constexpr int kClaimAhead = 6;          // blocks of wave 0 left when the next range is claimed
// LDS per workgroup: the merge buffer (16 KiB; two workgroups share a CU)
constexpr int kLdsFloats = kNW * kMaxG * kD;
static_assert(kLdsFloats >= kNW * kMaxG * kD, "merge buffer");
constexpr size_t kWsHeader = 256;       // the range counter; then the arrival counters, the partial states
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;           // log2-domain slack before the softmax reference moves

// gfx9-family buffer descriptor word 3 (raw 32-bit accesses, no swizzle)
constexpr int kBufferFlags = 0x00020000;

// Buffer loads.  CP is the cache policy: 0 the default, kStream the
// non-temporal hint (gfx950's NT bit): for tiles that a call reads exactly
// once, so they do not displace what the caches hold (measured on the
// long-context decode: 320 -> 297 us per call).  Tiles read again, by other
// waves or by the next call, keep the default.
constexpr int kStream = 2;
template <int CP = 0>
__device__ __forceinline__ uint4 ld_buf16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CP));
}
template <int CP = 0>
__device__ __forceinline__ uint2 ld_buf8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, CP));
}
template <int CP = 0>
__device__ __forceinline__ uint32_t ld_buf4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, CP);
}

// 16 bytes per lane from buffer rs at byte offset voff into LDS at lds + 16 * lane
// (gfx950 direct-to-LDS buffer load; lds is wave-uniform)
__device__ __forceinline__ void ld_buf_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}
// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// workgroup barrier without __syncthreads' fences (those would wait for
// every direct-to-LDS load in flight); callers wait for what must be done
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
// D = A B + C on 16 x 16 tiles.  Lane (j = lane / 16, r = lane % 16) holds
// row r of A and column r of B with the reduction elements of group j, and
// receives rows 4j..4j+3 of column r of D.
__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x16_bf16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// two E4M3FN codes (bytes 2 HI, 2 HI + 1 of w) -> a bf16 pair, exactly
// (every E4M3FN value is a bf16 value)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 c) {
  return make_uint4(fp8x2_to_bf16x2<false>(c.x), fp8x2_to_bf16x2<true>(c.x),
                    fp8x2_to_bf16x2<false>(c.y), fp8x2_to_bf16x2<true>(c.y));
}

struct DecodeKArgs {
  const uint16_t* q; int64_t q_stride;
  const uint8_t* k_cache; const uint8_t* v_cache; int num_blocks;   // bf16 or E4M3FN tiles
  const int32_t* block_tables; int max_blocks;
  const int32_t* context_lens; int num_seqs;
  uint16_t* out; int64_t out_stride;
  float* ws_acc;   // [2 R][G][128]: partial outputs (range r: slots 2r, 2r + 1)
  float* ws_ml;    // [2 R][G][2]:   reference max (log2 domain) and sum
  int num_heads, num_kv_heads, max_context_len;
  int tier_wgs[kTiers];   // most ranges per tier of the cascade's schedule (host bound on U)
  int num_ranges;         // ranges the workspace holds (every schedule's R is at most this)
  int* claim;             // [0] range counter: zero at launch
  int* arrive;            // [num_ranges] per range r: units arrived of the shared segment
                          // whose last unit is in r: zero at launch
  float scale_log2;   // scale * log2 e (* k_scale with an FP8 cache)
  float out_scale;    // 1, or v_scale with an FP8 cache
  // shared-prefix cascade (unused by the plain decode)
  int2* cas;              // per sequence: prefix blocks it skips, prefix chunks to fold in
  float* pre_ml;          // [chunk][S H][2]: prefix chunk states (reference max, sum)
  float* pre_acc;         // [chunk][S H][128]: prefix chunk partial outputs
  unsigned* err;          // the device error word (may be null)
};

// Context lengths are clamped to [1, max_context_len] (what the workspace
// was sized for); a value outside breaks the contract and makes that
// sequence's output NaN.
__device__ __forceinline__ int clamp_ctx(int c, int maxc) { return c < 1 ? 1 : (c > maxc ? maxc : c); }
__device__ __forceinline__ int nblocks_of(int c) { return (c + kBlk - 1) / kBlk; }
// blocks of sequence s that the stream kernel attends: all of them, or in a
// cascade those after the shared prefix (at least one)
template <bool CAS>
__device__ __forceinline__ int seg_blocks(const DecodeKArgs& a, int s) {
  const int n = nblocks_of(clamp_ctx(a.context_lens[s], a.max_context_len));
  if constexpr (CAS) return n - a.cas[s].x;
  return n;
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), l);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// U = Hkv * sum_s n_s (n_s = blocks of sequence s); the same in every lane
template <bool CAS>
__device__ int64_t total_units(const DecodeKArgs& a, int lane) {
  int64_t t = 0;
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int s = base + lane;
    const int n = s < a.num_seqs ? seg_blocks<CAS>(a, s) : 0;
    t += readlane64(wave_incl_scan(n, lane), 63);
  }
  return t * a.num_kv_heads;
}

// The unit u as (sequence s, KV head g, block b); n = blocks of s; the
// segment of (s, g) starts at unit seg0.  Every lane gets the same values.
struct Cursor {
  int s, g, b, n;
  int64_t seg0;
};
template <bool CAS>
__device__ Cursor locate(const DecodeKArgs& a, int64_t u, int lane) {
  const int Hkv = a.num_kv_heads;
  int64_t run = 0;                   // blocks of the sequences before this chunk
  Cursor c{0, 0, 0, 1, 0};
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int s = base + lane;
    const bool in = s < a.num_seqs;
    const int n = in ? seg_blocks<CAS>(a, s) : 0;
    const int64_t incl = run + wave_incl_scan(n, lane);        // blocks up to and with s
    const uint64_t hit = __builtin_amdgcn_ballot_w64(in && static_cast<int64_t>(Hkv) * incl > u);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      c.s = base + l;
      c.n = __builtin_amdgcn_readlane(n, l);
      const int64_t first = static_cast<int64_t>(Hkv) * (readlane64(incl, l) - c.n);
      const int64_t off = u - first;
      c.g = static_cast<int>(off / c.n);
      c.b = static_cast<int>(off - static_cast<int64_t>(c.g) * c.n);
      c.seg0 = first + static_cast<int64_t>(c.g) * c.n;
      return c;
    }
    run = readlane64(incl, 63);
  }
  return c;   // not reached for u < U
}

// The ranges per tier for the batch's U units.  With one tier R is at most
// kCUs + 2, below the host's three-tier bound for any U >= kOneTierUnits.
struct Schedule {
  int n[kTiers];
  int pct[kTiers + 1];
  int R;
};
template <bool CAS, bool F8>
__device__ Schedule schedule_for(const DecodeKArgs& a, int64_t U) {
  Schedule sc;
  sc.R = 0;
  if constexpr (!CAS) {
    // one tier of equal ranges; tiers 1 and 2 hold one empty range each,
    // and the host's bound a.num_ranges covers every R this gives
    for (int t = 0; t <= kTiers; ++t) sc.pct[t] = kOneTierPct[t];
    const int cap = min(!F8 && U >= kBf16WideUnits ? kCUs : kPlainRanges, a.num_ranges - (kTiers - 1));
    const int64_t n = (U + kOneTierMin - 1) / kOneTierMin;
    sc.n[0] = static_cast<int>(n < 1 ? 1 : (n > cap ? cap : n));
    for (int t = 1; t < kTiers; ++t) sc.n[t] = 1;
    for (int t = 0; t < kTiers; ++t) sc.R += sc.n[t];
    return sc;
  }
  const int* pct = U >= kOneTierUnits ? kOneTierPct : kTierPct;
  for (int t = 0; t <= kTiers; ++t) sc.pct[t] = pct[t];
  for (int t = 0; t < kTiers; ++t) {
    const int64_t share = U * sc.pct[t + 1] / 100 - U * sc.pct[t] / 100;
    const int64_t n = (share + kTierMin[t] - 1) / kTierMin[t];
    sc.n[t] = static_cast<int>(n < 1 ? 1 : (n > a.tier_wgs[t] ? a.tier_wgs[t] : n));
    sc.R += sc.n[t];
  }
  return sc;
}
// First unit of range r (r = R gives U).
__device__ int64_t range_begin(const Schedule& sc, int64_t r, int64_t U) {
  int64_t first = 0;
#pragma unroll
  for (int t = 0; t < kTiers; ++t) {
    const int n = sc.n[t];
    const int64_t b0 = U * sc.pct[t] / 100, b1 = U * sc.pct[t + 1] / 100;
    if (r < first + n) return b0 + (r - first) * (b1 - b0) / n;
    first += n;
  }
  return U;
}
// The range that holds unit u < U (ranges may be empty; this is the one
// whose [begin, end) contains u).
__device__ int64_t range_of(const Schedule& sc, int64_t u, int64_t U) {
  int64_t first = 0;
#pragma unroll
  for (int t = 0; t < kTiers; ++t) {
    const int n = sc.n[t];
    const int64_t b0 = U * sc.pct[t] / 100, b1 = U * sc.pct[t + 1] / 100;
    if (u < b1) return first + ((u - b0 + 1) * n - 1) / (b1 - b0);
    first += n;
  }
  return first - 1;
}

// Cascade: fold the shared-prefix chunk states of (sequence s, query head
// qh) into a state (M, L, o) of its private keys (log2 domain, M finite):
//   M' = max(M, m_c),  L' = L 2^(M - M') + sum_c l_c 2^(m_c - M'),  o' likewise.
// Chunks are loaded kFoldBatch at a time, all loads of a batch in flight.
constexpr int kFoldBatch = 8;
__device__ __forceinline__ void fold_prefix(const DecodeKArgs& a, int s, int qh, int e, float& M,
                                            float& L, float& o) {
  const int nc = a.cas[s].y;
  const int64_t row = static_cast<int64_t>(s) * a.num_heads + qh;
  const int64_t cstride = static_cast<int64_t>(a.num_seqs) * a.num_heads;
  for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
    float pm[kFoldBatch], pl[kFoldBatch], pv[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const int64_t r = (c0 + i < nc ? c0 + i : c0) * cstride + row;
      pm[i] = a.pre_ml[r * 2];
      pl[i] = a.pre_ml[r * 2 + 1];
      pv[i] = a.pre_acc[r * kD + e];
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i)
      if (c0 + i < nc) Mn = fmaxf(Mn, pm[i]);
    const float f = __builtin_amdgcn_exp2f(M - Mn);
    L *= f;
    o *= f;
    M = Mn;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      if (c0 + i < nc) {
        const float wt = __builtin_amdgcn_exp2f(pm[i] - M);
        L = fmaf(pl[i], wt, L);
        o = fmaf(pv[i], wt, o);
      }
    }
  }
}

// fold_prefix for four consecutive dims e0 .. e0 + 3 of one state: the
// chunks' (max, sum) are loaded once for the four, and each dim's arithmetic
// is fold_prefix's
__device__ __forceinline__ void fold_prefix4(const DecodeKArgs& a, int s, int qh, int e0, float& M,
                                             float& L, float4& o) {
  const int nc = a.cas[s].y;
  const int64_t row = static_cast<int64_t>(s) * a.num_heads + qh;
  const int64_t cstride = static_cast<int64_t>(a.num_seqs) * a.num_heads;
  for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
    float pm[kFoldBatch], pl[kFoldBatch];
    float4 pv[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const int64_t r = (c0 + i < nc ? c0 + i : c0) * cstride + row;
      pm[i] = a.pre_ml[r * 2];
      pl[i] = a.pre_ml[r * 2 + 1];
      pv[i] = *reinterpret_cast<const float4*>(a.pre_acc + r * kD + e0);
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i)
      if (c0 + i < nc) Mn = fmaxf(Mn, pm[i]);
    const float f = __builtin_amdgcn_exp2f(M - Mn);
    L *= f;
    o.x *= f; o.y *= f; o.z *= f; o.w *= f;
    M = Mn;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      if (c0 + i < nc) {
        const float wt = __builtin_amdgcn_exp2f(pm[i] - M);
        L = fmaf(pl[i], wt, L);
        o.x = fmaf(pv[i].x, wt, o.x);
        o.y = fmaf(pv[i].y, wt, o.y);
        o.z = fmaf(pv[i].z, wt, o.z);
        o.w = fmaf(pv[i].w, wt, o.w);
      }
    }
  }
}

// Device-coherent (agent scope) accesses to the partial states: they reach
// or read the point where every XCD's accesses meet (gfx950's SC1 bit), so
// a state one workgroup stores and waits for is what a workgroup on any XCD
// loads after the arrival counter says it is there.
constexpr int kCoherent = 16;           // buffer-load cache policy: SC1
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Range r holds units [range_begin(r), range_begin(r + 1)); a tier with at
// least one unit has at least as many units as ranges, so only a tier
// without units has an empty range (its only one).  Bit t: tier t has units.
__device__ __forceinline__ unsigned live_tiers(const Schedule& sc, int64_t U) {
  unsigned m = 0;
#pragma unroll
  for (int t = 0; t < kTiers; ++t)
    if (U * sc.pct[t + 1] / 100 > U * sc.pct[t] / 100) m |= 1u << t;
  return m;
}

// Merge of shared segment (s, g), units [seg0, seg0 + n), by the workgroup
// whose range completed it.  Its pieces are the partial states of the
// non-empty ranges ra..rb that hold its units: ra's piece is ra's first
// (slot 2 ra) if ra begins with the segment, else ra's last (slot 2 ra + 1);
// every later range's piece is its first (slot 2 r).  Thread (head h, dims
// 4 e4 .. 4 e4 + 3) merges them in range order, kMergeBatch at a time with
// every load of a batch in flight:
//   M = max_r m_r,  L = sum_r l_r 2^(m_r - M),  o = sum_r a_r 2^(m_r - M) / L
// The result depends only on the logical sizes: bitwise reproducible.
constexpr int kMergeBatch = 16;
template <int G, bool CAS>
__device__ __forceinline__ void merge_segment(const DecodeKArgs& a, const Schedule& sc, int64_t U,
                                              int s, int g, int64_t seg0, int n, int tid) {
  if (tid >= G * (kD / 4)) return;
  const int h = tid / (kD / 4), e4 = tid % (kD / 4);
  const int64_t ra = range_of(sc, seg0, U), rb = range_of(sc, seg0 + n - 1, U);
  const bool ra_first = range_begin(sc, ra, U) == seg0;
  const unsigned tiers = live_tiers(sc, U);
  const int64_t n0 = sc.n[0], n01 = n0 + sc.n[1];
  float M = -INFINITY, L = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const auto racc = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_acc, static_cast<short>(0), 2 * a.num_ranges * G * kD * 4, kBufferFlags);
  for (int64_t x0 = ra; x0 <= rb; x0 += kMergeBatch) {
    float pm[kMergeBatch], pl[kMergeBatch];
    float4 v[kMergeBatch];
    bool live[kMergeBatch];
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
      // loads only for pieces of the segment (x0 + q <= rb is uniform)
      const int64_t x = x0 + q;
      live[q] = x <= rb && (x == ra || ((tiers >> (x < n0 ? 0 : x < n01 ? 1 : 2)) & 1u));
      if (live[q]) {
        const int64_t sb = (2 * x + (x == ra && !ra_first ? 1 : 0)) * G + h;
        pm[q] = load_coherent(&a.ws_ml[sb * 2]);
        pl[q] = load_coherent(&a.ws_ml[sb * 2 + 1]);
        v[q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                              racc, static_cast<int>((sb * (kD / 4) + e4) * 16), 0,
                                              kCoherent));
      } else {
        pm[q] = pl[q] = 0.0f;
        v[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    float Mc = M;
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q)
      if (live[q]) Mc = fmaxf(Mc, pm[q]);
    if (Mc > M) {                        // rescale the running sums (M = -inf: they are 0)
      const float f = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mc);
      L *= f;
      o.x *= f; o.y *= f; o.z *= f; o.w *= f;
      M = Mc;
    }
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
      if (live[q]) {
        const float wt = __builtin_amdgcn_exp2f(pm[q] - M);
        L = fmaf(pl[q], wt, L);
        o.x = fmaf(v[q].x, wt, o.x);
        o.y = fmaf(v[q].y, wt, o.y);
        o.z = fmaf(v[q].z, wt, o.z);
        o.w = fmaf(v[q].w, wt, o.w);
      }
    }
  }
  const int qh = g * G + h;
  if constexpr (CAS) fold_prefix4(a, s, qh, 4 * e4, M, L, o);
  const float os = a.out_scale;
  uint2 w;
  w.x = pack_bf16x2(o.x * os / L, o.y * os / L);
  w.y = pack_bf16x2(o.z * os / L, o.w * os / L);
  *reinterpret_cast<uint2*>(a.out + static_cast<int64_t>(s) * a.out_stride +
                            static_cast<int64_t>(qh) * kD + 4 * e4) = w;
}

// F8: the caches hold E4M3FN codes (K tile 2 KiB, V tile 2 KiB); they are
// widened to bf16 in registers and the same arithmetic follows.
// CAS: a cascade's private level (each sequence's keys after its shared
// prefix; the prefix chunk states are folded in where a segment's output is
// written).
// BS: cache blocks of 16 << BS tokens.  The work units stay 16-token blocks:
// unit b of a sequence is sub-block b % 2^BS of its table entry b >> BS,
// whose K rows are contiguous and whose V rows are 16-key runs of the
// longer dims rows of the [d][16 << BS] tile.
template <int G, bool F8, bool CAS, int BS>
__global__ __launch_bounds__(kThreads, 2) void decode_stream_kernel(DecodeKArgs a) {
  constexpr int kEl = F8 ? 1 : 2;                 // bytes per cache element
  constexpr int kTileBytes = kBlk * kD * kEl;     // one 16-token (sub-)tile of K or V
  constexpr int kBS = kBlk << BS;                 // tokens per cache block
  constexpr int kVRange = (127 * kBS + kBlk) * kEl;   // V bytes from a sub-tile's start
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int Hkv = a.num_kv_heads;
  const int64_t U = total_units<CAS>(a, lane);
  const Schedule sched = schedule_for<CAS, F8>(a, U);

  // per-wave softmax states of a piece, merged at its end
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
  float (*sacc)[kMaxG * kD] = reinterpret_cast<float (*)[kMaxG * kD]>(lds);
  __shared__ float sm[kNW][kMaxG], sl[kNW][kMaxG];
  __shared__ int sbad[kNW];
  __shared__ int s_next, s_merge;

  // MFMA lane roles: lane group j4, column (query head, or row of the A
  // operand) r16
  const int r16 = lane & 15;
  const int j4 = lane >> 4;
  // K: key r16, bytes 64 c + 16 j4 of its row (bf16: c < 4; FP8: c < 2).
  // V: dim 16 t + r16, keys 4 j4 .. 4 j4 + 3 (bf16: 8 bytes; FP8: 4 bytes).
  constexpr int kKLoads = F8 ? 2 : 4;
  const int koff = r16 * kD * kEl + j4 * 16;
  const int voff = (r16 * kBS + j4 * 4) * kEl;
  using VWord = typename std::conditional<F8, uint32_t, uint2>::type;
  const float c = a.scale_log2;

  // Workgroup i takes range i first; later ranges are claimed in order
  // (gridDim.x + the counter), each a few blocks before the current range
  // ends (by thread 0), so its latency is hidden but a workgroup never holds
  // a range it has not nearly reached.
  int rg = blockIdx.x;
  while (rg < sched.R) {
  int next = 0;
  bool claimed = false;
  const int64_t u0 = range_begin(sched, rg, U), u1 = range_begin(sched, rg + 1, U);
  if (u0 < u1) {
  Cursor cur = locate<CAS>(a, u0, lane);
  int64_t u = u0;
  bool first_piece = true;
  while (true) {
    // ---- one piece: blocks [b0, b0 + cnt) of segment (s, g); this wave
    // takes blocks b0 + wave + kNW i, i < nbw ----
    const int s = cur.s, g = cur.g, b0 = cur.b, n = cur.n;
    const int cnt = static_cast<int>(min(static_cast<int64_t>(n - b0), u1 - u));
    const int nbw = cnt > wave ? (cnt - wave + kNW - 1) / kNW : 0;
    const int ctx_raw = a.context_lens[s];
    // error flags of the piece (wave-uniform), reported once at its end
    unsigned bad = ctx_raw < 1 || ctx_raw > a.max_context_len ? kErrSequence : 0u;
    const int ctx = clamp_ctx(ctx_raw, a.max_context_len);
    const int kb0 = b0 + (CAS ? a.cas[s].x : 0);   // the piece's first 16-token block
    const int vb0 = kb0 + wave;                      // this wave's first 16-token block
    const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

    // this wave's block ids, 64 at a time: lane i of ids_c holds its block
    // cbase + i, of ids_n its block cbase + 64 + i (table entries; with
    // longer cache blocks consecutive 16-token blocks share an entry)
    int cbase = 0;
    int ids_c = lane < nbw ? bt[(vb0 + kNW * lane) >> BS] : 0;
    int ids_n = 64 + lane < nbw ? bt[(vb0 + kNW * (64 + lane)) >> BS] : 0;

    // q as the B operand in the dim order of the K pieces: chunk cc (32
    // dims) of lane (j4, head r16) holds dims 32 cc + 8 j4 .. (bf16 cache) or
    // 64 (cc / 2) + 16 j4 + 8 (cc % 2) .. (FP8 cache); padding heads are zero
    uint4 qf[4];
    {
      const uint16_t* qp = a.q + static_cast<int64_t>(s) * a.q_stride +
                           static_cast<int64_t>(g * G + r16) * kD;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int d = F8 ? (cc >> 1) * 64 + j4 * 16 + (cc & 1) * 8 : cc * 32 + j4 * 8;
        qf[cc] = r16 < G ? *reinterpret_cast<const uint4*>(qp + d) : make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // Tiles are read with buffer loads through a per-tile descriptor
    // (uniform, in SGPRs).  Every pipeline load is issued unconditionally so
    // the number of loads in flight is static; a prefetch past the wave's
    // last block gets a zero-size descriptor, which returns zeros without
    // touching memory.  An id outside the pool marks the piece bad and
    // reads block 0 instead.
    auto issue = [&](int i, uint4 (&kb)[kKLoads], VWord (&vb)[8]) {
      const bool live = i < nbw;
      int id = 0;
      if (live) {
        const int k = i - cbase;
        id = k < 64 ? __builtin_amdgcn_readlane(ids_c, k) : __builtin_amdgcn_readlane(ids_n, k - 64);
        if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) {
          bad |= kErrBlock;
          id = 0;
        }
      }
      const int sub = (vb0 + kNW * i) & ((1 << BS) - 1);   // 16-token sub-block of the entry
      const int64_t tile = (static_cast<int64_t>(id) * Hkv + g) * (kTileBytes << BS);
      const auto rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.k_cache + tile + sub * kTileBytes), static_cast<short>(0),
          live ? kTileBytes : 0, kBufferFlags);
      const auto rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.v_cache + tile + sub * kBlk * kEl), static_cast<short>(0),
          live ? kVRange : 0, kBufferFlags);
#pragma unroll
      for (int cc = 0; cc < kKLoads; ++cc) kb[cc] = ld_buf16<kStream>(rk, koff + cc * 64);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if constexpr (F8)
          vb[t] = ld_buf4<kStream>(rv, voff + t * 16 * kBS);
        else
          vb[t] = ld_buf8<kStream>(rv, voff + t * 16 * kBS * 2);
      }
    };

    // Online softmax state per query head (column r16): ms is the reference
    // maximum in the log2 domain (raw max * scale * log2 e), l the lane's
    // share of the sum of the rounded p, acc the 16 x 128 output tile
    // (lane: head r16, dims 16 t + 4 j4 + e).
    float ms = -INFINITY, l = 0.0f;
    f32x4_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = {0.0f, 0.0f, 0.0f, 0.0f};

    auto block = [&](int i, const uint4 (&kb)[kKLoads], VWord (&vb)[8]) {
      // S^T = K q^T: lane (j4, r16) gets head r16's scores of keys 4 j4 + e
      f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint4 kf;
        if constexpr (F8)
          kf = fp8x8_to_bf16x8((cc & 1) ? make_uint2(kb[cc >> 1].z, kb[cc >> 1].w)
                                        : make_uint2(kb[cc >> 1].x, kb[cc >> 1].y));
        else
          kf = kb[cc];
        sc = mfma_16x16x32_bf16(kf, qf[cc], sc);
      }
      // keys past the context (slots there may hold NaN) are excluded by select
      const int t0 = (kb0 + wave + kNW * i) * kBlk + j4 * 4;
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = t0 + e < ctx ? sc[e] : -INFINITY;
      float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      // every block has a key inside the context, so bm is finite
      const float bms = bm * c;
      const bool up = bms > ms + kLazy;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float alpha = up ? __builtin_amdgcn_exp2f(ms - bms) : 1.0f;
        ms = up ? bms : ms;
        l *= alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] *= alpha;
      }
      // p = 2^(z * scale * log2 e - ms), rounded to bf16: the B operand of
      // P V (keys 4 j4 + e, head r16); the normaliser sums the rounded values
      const float nm = -ms;
      uint2 p;
      p.x = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(z[0], c, nm)),
                        __builtin_amdgcn_exp2f(fmaf(z[1], c, nm)));
      p.y = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(z[2], c, nm)),
                        __builtin_amdgcn_exp2f(fmaf(z[3], c, nm)));
      l += (bf16_lo(p.x) + bf16_hi(p.x)) + (bf16_lo(p.y) + bf16_hi(p.y));
      // O^T += V^T P^T, 16 dims per MFMA
      uint2 vf[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if constexpr (F8)
          vf[t] = make_uint2(fp8x2_to_bf16x2<false>(vb[t]), fp8x2_to_bf16x2<true>(vb[t]));
        else
          vf[t] = vb[t];
      }
      if (t0 + 4 > ctx) {                // last block: tail slots may hold NaN
        const uint32_t m0 = t0 >= ctx ? 0u : (t0 + 1 >= ctx ? 0xffffu : 0xffffffffu);
        const uint32_t m1 = t0 + 2 >= ctx ? 0u : (t0 + 3 >= ctx ? 0xffffu : 0xffffffffu);
#pragma unroll
        for (int t = 0; t < 8; ++t) vf[t] = make_uint2(vf[t].x & m0, vf[t].y & m1);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = mfma_16x16x16_bf16(vf[t], p, acc[t]);
    };

    {
      // wave 0 claims the next range kClaimAhead of its blocks before the
      // end of the range's last piece
      const int claim_at = u + cnt >= u1 && wave == 0 ? max(0, nbw - kClaimAhead) : -1;
      uint4 kb[kNBuf][kKLoads];
      VWord vb[kNBuf][8];
#pragma unroll
      for (int j = 0; j < kNBuf - 1; ++j) issue(j, kb[j], vb[j]);
      for (int i = 0; i < nbw; i += kNBuf) {
#pragma unroll
        for (int j = 0; j < kNBuf; ++j) {
          if (i + j == claim_at) {
            if (lane == 0) next = gridDim.x + atomicAdd(a.claim, 1);
            claimed = true;
          }
          if (i + j == cbase + 64 && i + j < nbw) {   // next 64 ids; the window covers the prefetch
            cbase += 64;
            ids_c = ids_n;
            ids_n = cbase + 64 + lane < nbw ? bt[(vb0 + kNW * (cbase + 64 + lane)) >> BS] : 0;
          }
          issue(i + j + kNBuf - 1, kb[(j + kNBuf - 1) % kNBuf], vb[(j + kNBuf - 1) % kNBuf]);
          if (i + j < nbw) block(i + j, kb[j], vb[j]);
        }
      }
    }

    // ---- merge of the waves' states: the piece's result ----
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (r16 < G) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<float4*>(&sacc[wave][r16 * kD + t * 16 + j4 * 4]) =
            make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
      if (j4 == 0) {
        sm[wave][r16] = ms;              // -inf for a wave without blocks
        sl[wave][r16] = l;
      }
    }
    if (lane == 0) sbad[wave] = static_cast<int>(bad);
    __syncthreads();
    unsigned pflags = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) pflags |= static_cast<unsigned>(sbad[w]);
    const bool pbad = pflags != 0;
    if (pbad && tid == 0) report_error(a.err, pflags);
    const bool whole = b0 == 0 && cnt == n;
    const int64_t slot = 2 * static_cast<int64_t>(rg) + (first_piece ? 0 : 1);
    for (int idx = tid; idx < G * kD; idx += kThreads) {
      const int h = idx / kD, e = idx % kD;
      float M = sm[0][h];
#pragma unroll
      for (int w = 1; w < kNW; ++w) M = fmaxf(M, sm[w][h]);
      float v = 0.0f, L = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(sm[w][h] - M);   // 0 for a wave without blocks
        v = fmaf(sacc[w][idx], wt, v);
        L = fmaf(sl[w][h], wt, L);
      }
      if (whole) {                       // the whole segment: final output
        const int qh = g * G + h;
        if constexpr (CAS) fold_prefix(a, s, qh, e, M, L, v);
        a.out[static_cast<int64_t>(s) * a.out_stride + static_cast<int64_t>(qh) * kD + e] =
            f32_to_bf16(pbad ? __builtin_nanf("") : v * a.out_scale / L);
      } else {                           // a share of the segment: partial state
        store_coherent(&a.ws_acc[(slot * G + h) * kD + e], v);
        if (e == 0) {
          store_coherent(&a.ws_ml[(slot * G + h) * 2], M);
          store_coherent(&a.ws_ml[(slot * G + h) * 2 + 1], pbad ? __builtin_nanf("") : L);
        }
      }
    }
    if (!whole) {
      // a share of segment (s, g): once every thread's partial-state stores
      // are complete, add its units to the arrival counter of the range
      // that holds the segment's last unit; the range whose units complete
      // the segment merges it.  The states are stored and read with
      // device-coherent accesses (each XCD has its own L2); fences would
      // write back and invalidate whole L2s (measured: the Qwen3-0.6B-shaped
      // decode 38 -> 205 us).
      const int64_t seg0 = u - b0;
      const int64_t rb = range_of(sched, seg0 + n - 1, U);
      wait_vmcnt<0>();
      __syncthreads();
      if (tid == 0) s_merge = atomicAdd(a.arrive + rb, cnt) + cnt == n;
      __syncthreads();
      if (s_merge) merge_segment<G, CAS>(a, sched, U, s, g, seg0, n, tid);
    }
    u += cnt;
    if (u >= u1) break;
    __syncthreads();                     // the merge buffers are reused by the next piece
    first_piece = false;
    cur.b = 0;
    if (++cur.g == Hkv) {
      cur.g = 0;
      ++cur.s;
      cur.n = seg_blocks<CAS>(a, cur.s);
    }
  }
  }
  if (tid == 0) s_next = claimed ? next : gridDim.x + atomicAdd(a.claim, 1);
  __syncthreads();                       // s_next is written; the merge buffers are free
  rg = s_next;
  __syncthreads();                       // every thread has read s_next
  }
}

// ---- shared-prefix cascade: the prefix level ----
//
// Group p's members are seqs[indptr[p] .. indptr[p + 1]); its prefix is the
// first lens[p] tokens (whole blocks) of each, held in the same physical
// blocks, which are read through the first member's block table.  The
// group's (member, query head) pairs of KV head g form cols = members x G
// columns; column col is member col / G, query head g G + col % G.  The
// prefix blocks are cut into chunks of chunk_blocks; task (p, g, chunk) x
// four column tiles is one workgroup, wave w taking the 16 columns
// 16 (4 xc + w) .. of the tile group xc.  Each wave attends its 16 columns to
// the chunk's blocks with the decode's tile math (S^T = K Q^T, lazy online
// softmax, O^T += V^T P^T); only the 16 columns now belong to 16 different
// (sequence, head) pairs, so no MFMA column is padding once a group has 16
// of them.  The chunk state (reference max, sum, partial output) goes to row
// chunk (S H) + s H + qh of the prefix state arrays.
//
// A group is attended only when it is well formed: 0 < lens[p] <= the
// host's max_prefix_len, whole blocks, first member in range with a key after
// the prefix.  A member gets the cascade (cas[s] = (prefix blocks, chunks))
// only when its group is attended and it has a key after the prefix;
// every other sequence is decoded over its whole table.
struct CascadeArgs {
  const int32_t* indptr;   // [P + 1]
  const int32_t* seqs;     // [members]
  const int32_t* lens;     // [P] prefix tokens
  int num_prefixes, num_members, max_prefix_len;
  int chunk_blocks, max_chunks, col_wgs;
};

// the group's prefix in 16-token blocks (0: the group is not attended)
template <int BS>
__device__ __forceinline__ int group_prefix_blocks(const DecodeKArgs& a, const CascadeArgs& ca,
                                                   int p) {
  const int L = ca.lens[p];
  if (L <= 0 || L > ca.max_prefix_len || L % (kBlk << BS)) return 0;
  const int i0 = ca.indptr[p];
  if (i0 < 0 || i0 >= ca.num_members || ca.indptr[p + 1] <= i0 ||
      ca.indptr[p + 1] > ca.num_members)
    return 0;
  const int s0 = ca.seqs[i0];
  if (s0 < 0 || s0 >= a.num_seqs) return 0;
  const int PB = L / kBlk;
  return PB < nblocks_of(clamp_ctx(a.context_lens[s0], a.max_context_len)) ? PB : 0;
}

// workgroup 0: zero the range and job counters and set cas[] for the
// private level
template <int BS>
__device__ void cascade_prep(const DecodeKArgs& a, const CascadeArgs& ca) {
  const int tid = threadIdx.x;
  if (tid == 0) a.claim[0] = 0;
  for (int r = tid; r < a.num_ranges; r += kThreads) a.arrive[r] = 0;
  for (int s = tid; s < a.num_seqs; s += kThreads) a.cas[s] = make_int2(0, 0);
  __syncthreads();
  for (int i = tid; i < ca.num_members; i += kThreads) {
    // the group of member i: the last p with indptr[p] <= i
    int lo = 0, hi = ca.num_prefixes - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ca.indptr[mid] <= i) lo = mid; else hi = mid - 1;
    }
    if (ca.indptr[lo] > i || ca.indptr[lo + 1] <= i) continue;
    const int PB = group_prefix_blocks<BS>(a, ca, lo);
    const int s = ca.seqs[i];
    if (PB == 0 || s < 0 || s >= a.num_seqs) continue;
    if (PB >= nblocks_of(clamp_ctx(a.context_lens[s], a.max_context_len))) continue;
    a.cas[s] = make_int2(PB, (PB + ca.chunk_blocks - 1) / ca.chunk_blocks);
  }
}

template <int G, bool F8, int BS>
__global__ __launch_bounds__(kThreads, 2) void decode_prefix_kernel(DecodeKArgs a, CascadeArgs ca) {
  if (blockIdx.x == 0) {
    cascade_prep<BS>(a, ca);
    return;
  }
  constexpr int kEl = F8 ? 1 : 2;
  constexpr int kTileBytes = kBlk * kD * kEl;     // one 16-token (sub-)tile of K or V
  constexpr int kBS = kBlk << BS;                 // tokens per cache block
  constexpr int kVRange = (127 * kBS + kBlk) * kEl;   // V bytes from a sub-tile's start
  constexpr int kKLoads = F8 ? 2 : 4;
  using VWord = typename std::conditional<F8, uint32_t, uint2>::type;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int r16 = lane & 15, j4 = lane >> 4;
  // Tasks in the order (column tile xc, group p, KV head g, chunk), the
  // column tile slowest.  The host sizes the column tiles for all members in
  // one group, so with several groups most tiles past the first few find no
  // column of their group: they leave after one round of loads (the group's
  // member range), and coming last in the grid they do so while the live
  // workgroups finish instead of holding CU slots among them (measured: the
  // shared-prompt cascade 98.5 -> 85.2 us against the tile fastest).
  const int task = blockIdx.x - 1;
  const int ny = ca.num_prefixes * a.num_kv_heads * ca.max_chunks;
  const int xc = task / ny;
  int y = task - xc * ny;
  const int chunk = y % ca.max_chunks;
  y /= ca.max_chunks;
  const int g = y % a.num_kv_heads;
  const int p = y / a.num_kv_heads;
  const int i0 = ca.indptr[p];
  const int cols = (ca.indptr[p + 1] - i0) * G;
  if (xc * kNW * 16 >= cols) return;                   // uniform per workgroup
  const int PB = group_prefix_blocks<BS>(a, ca, p);
  const int col0 = (xc * kNW + wave) * 16;
  const int bb = chunk * ca.chunk_blocks;
  const int be = min(PB, bb + ca.chunk_blocks);
  if (PB == 0 || bb >= be) return;                     // uniform per workgroup
  const int nb = be - bb;                              // <= 64 blocks
  // a wave whose 16 columns all lie past the group's pairs computes nothing
  // (with bf16 tiles it still loads its share of the workgroup's tiles)
  const bool wave_live = col0 < cols;                  // wave-uniform
  if constexpr (F8) {
    if (!wave_live) return;
  }

  // this lane's column: (member sequence s, query head qh)
  const int col = col0 + r16;
  int s = col < cols ? ca.seqs[i0 + col / G] : -1;
  if (s >= a.num_seqs) s = -1;
  const int qh = g * G + col % G;
  uint4 qf[4];
  {
    const uint16_t* qp = a.q + static_cast<int64_t>(s < 0 ? 0 : s) * a.q_stride +
                         static_cast<int64_t>(qh) * kD;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int d = F8 ? (cc >> 1) * 64 + j4 * 16 + (cc & 1) * 8 : cc * 32 + j4 * 8;
      qf[cc] = s >= 0 ? *reinterpret_cast<const uint4*>(qp + d) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // the chunk's block ids, lane i holding (the table entry of) 16-token block bb + i
  const int s0 = ca.seqs[i0];
  const int ids =
      lane < nb ? a.block_tables[static_cast<int64_t>(s0) * a.max_blocks + ((bb + lane) >> BS)] : 0;
  const float c = a.scale_log2;
  bool bad = false;

  float ms = -INFINITY, l = 0.0f;
  f32x4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = {0.0f, 0.0f, 0.0f, 0.0f};

  // every prefix key lies inside every member's context: no masking.
  // kf(cc): the K operand of dims chunk cc; vf(t): the V operand of dims 16 t ..
  auto block = [&](auto&& kf, auto&& vf) __attribute__((always_inline)) {
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) sc = mfma_16x16x32_bf16(kf(cc), qf[cc], sc);
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float bms = bm * c;
    const bool up = bms > ms + kLazy;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float alpha = up ? __builtin_amdgcn_exp2f(ms - bms) : 1.0f;
      ms = up ? bms : ms;
      l *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    }
    const float nm = -ms;
    uint2 pp;
    pp.x = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[0], c, nm)),
                       __builtin_amdgcn_exp2f(fmaf(sc[1], c, nm)));
    pp.y = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[2], c, nm)),
                       __builtin_amdgcn_exp2f(fmaf(sc[3], c, nm)));
    l += (bf16_lo(pp.x) + bf16_hi(pp.x)) + (bf16_lo(pp.y) + bf16_hi(pp.y));
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = mfma_16x16x16_bf16(vf(t), pp, acc[t]);
  };

  if constexpr (F8) {
    // FP8 tiles: each wave reads its tiles into registers (codes widened to
    // bf16 there), two blocks in flight
    const int koff = r16 * kD * kEl + j4 * 16;
    const int voff = (r16 * kBS + j4 * 4) * kEl;
    auto issue = [&](int i, uint4 (&kb)[kKLoads], VWord (&vb)[8]) {
      const bool live = i < nb;
      int id = live ? __builtin_amdgcn_readlane(ids, i) : 0;
      if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) {
        bad = true;
        id = 0;
      }
      const int sub = (bb + i) & ((1 << BS) - 1);
      const int64_t tile = (static_cast<int64_t>(id) * a.num_kv_heads + g) * (kTileBytes << BS);
      const auto rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.k_cache + tile + sub * kTileBytes), static_cast<short>(0),
          live ? kTileBytes : 0, kBufferFlags);
      const auto rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.v_cache + tile + sub * kBlk * kEl), static_cast<short>(0),
          live ? kVRange : 0, kBufferFlags);
#pragma unroll
      for (int cc = 0; cc < kKLoads; ++cc) kb[cc] = ld_buf16(rk, koff + cc * 64);
#pragma unroll
      for (int t = 0; t < 8; ++t) vb[t] = ld_buf4(rv, voff + t * 16 * kBS);
    };
    auto run = [&](const uint4 (&kb)[kKLoads], const VWord (&vb)[8]) {
      block([&](int cc) {
              return fp8x8_to_bf16x8((cc & 1) ? make_uint2(kb[cc >> 1].z, kb[cc >> 1].w)
                                              : make_uint2(kb[cc >> 1].x, kb[cc >> 1].y));
            },
            [&](int t) {
              return make_uint2(fp8x2_to_bf16x2<false>(vb[t]), fp8x2_to_bf16x2<true>(vb[t]));
            });
    };
    uint4 kb0[kKLoads], kb1[kKLoads];
    VWord vb0[8], vb1[8];
    issue(0, kb0, vb0);
    for (int i = 0; i < nb; i += 2) {
      issue(i + 1, kb1, vb1);
      run(kb0, vb0);
      issue(i + 2, kb0, vb0);
      if (i + 1 < nb) run(kb1, vb1);
    }
  } else {
    // bf16 tiles go through an LDS ring of kPS blocks shared by the
    // workgroup's four waves (the four column tiles of the same blocks):
    // each block is read from L2/HBM once per workgroup, and kPS - 1 blocks
    // are in flight.  Stage layout (8 KiB): K tile [16 keys][256 B] with the
    // 16-byte chunks of key r at positions chunk ^ r; V tile [128 dims][32 B]
    // with the 16-byte halves of dim d at half ^ ((d >> 3) & 1).  Direct-to-
    // LDS loads (lane i's 16 bytes land at base + 16 i) fetch, per lane, the
    // source chunk that its slot holds.  Wave w issues K load w (keys 4w ..
    // 4w + 3) and V load w (dims 32 w .. 32 w + 31) of every block.
    constexpr int kPS = 8;
    constexpr int kStageBytes = 2 * kTileBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kPS * kStageBytes];
    const int kr = 4 * wave + (lane >> 4), kp = lane & 15;        // K slot of this lane's load
    const int ksrc = kr * (kD * 2) + ((kp ^ kr) & 15) * 16;
    const int vd = 32 * wave + (lane >> 1), vq = lane & 1;        // V slot of this lane's load
    const int vsrc = vd * (kBS * 2) + ((vq ^ (vd >> 3)) & 1) * 16;
    auto issue = [&](int i) __attribute__((always_inline)) {
      const bool live = i < nb;
      int id = live ? __builtin_amdgcn_readlane(ids, i) : 0;
      if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) {
        bad = true;
        id = 0;
      }
      const int sub = (bb + i) & ((1 << BS) - 1);
      const int64_t tile = (static_cast<int64_t>(id) * a.num_kv_heads + g) * (kTileBytes << BS);
      const auto rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.k_cache + tile + sub * kTileBytes), static_cast<short>(0),
          live ? kTileBytes : 0, kBufferFlags);
      const auto rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.v_cache + tile + sub * kBlk * 2), static_cast<short>(0),
          live ? kVRange : 0, kBufferFlags);
      uint8_t* st = ring + (i % kPS) * kStageBytes;
      ld_buf_lds16(rk, st + wave * 1024, ksrc);
      ld_buf_lds16(rv, st + kTileBytes + wave * 1024, vsrc);
    };
    // MFMA operands from a stage: K of key r16, 16-byte chunk 4 cc + j4;
    // V of dim 16 t + r16, keys 4 j4 .. 4 j4 + 3 (8 bytes)
    auto run = [&](int i) __attribute__((always_inline)) {
      const uint8_t* st = ring + (i % kPS) * kStageBytes;
      block([&](int cc) {
              return *reinterpret_cast<const uint4*>(st + r16 * (kD * 2) +
                                                     (((4 * cc + j4) ^ r16) & 15) * 16);
            },
            [&](int t) {
              const int d = 16 * t + r16;
              return *reinterpret_cast<const uint2*>(
                  st + kTileBytes + d * (kBlk * 2) + (((j4 >> 1) ^ (d >> 3)) & 1) * 16 +
                  (j4 & 1) * 8);
            });
    };
    // Block i: wait for this wave's loads of block i (2 loads per block;
    // those of the kPS - 2 later blocks may stay in flight), barrier (every
    // wave's loads of block i landed, and every wave is done with block
    // i - 1), refill that stage with block i + kPS - 1 (loads past the
    // chunk's end have empty ranges: zeros, no traffic), then the block.
#pragma unroll
    for (int i = 0; i < kPS - 1; ++i) issue(i);
    for (int i = 0; i < nb; ++i) {
      wait_vmcnt<2 * (kPS - 2)>();
      lds_barrier();
      issue(i + kPS - 1);
      if (wave_live) run(i);
    }
    wait_vmcnt<0>();
    if (!wave_live) return;
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (bad && lane == 0) report_error(a.err, kErrBlock);
  if (s >= 0) {
    const int64_t row = static_cast<int64_t>(chunk) * a.num_seqs * a.num_heads +
                        static_cast<int64_t>(s) * a.num_heads + qh;
    float* pa = a.pre_acc + row * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      *reinterpret_cast<float4*>(pa + t * 16 + j4 * 4) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    if (j4 == 0) {
      float* pm = a.pre_ml + row * 2;
      pm[0] = ms;
      pm[1] = bad ? __builtin_nanf("") : l;
    }
  }
}

// zero the range counter and the arrival counters
__global__ void decode_claim_reset_kernel(int* claim, int* arrive, int num_ranges) {
  if (threadIdx.x == 0) claim[0] = 0;
  for (int r = threadIdx.x; r < num_ranges; r += blockDim.x) arrive[r] = 0;
}

static size_t arrive_bytes(int num_ranges) { return (static_cast<size_t>(num_ranges) * 4 + 255) / 256 * 256; }

// ranges per tier for a batch of at most umax units
static void decode_schedule(int num_seqs, int max_context_len, int num_kv_heads, int (&wgs)[kTiers]) {
  const int64_t umax = static_cast<int64_t>(num_kv_heads) * num_seqs *
                       ((static_cast<int64_t>(max_context_len) + kBlk - 1) / kBlk);
  for (int t = 0; t < kTiers; ++t) {
    const int64_t share = umax * (kTierPctHost[t + 1] - kTierPctHost[t]) / 100;
    const int64_t n = (share + kTierMinHost[t] - 1) / kTierMinHost[t];
    wgs[t] = static_cast<int>(n < 1 ? 1 : (n > kTierWgs[t] ? kTierWgs[t] : n));
  }
}

// The ranges the workspace holds: the cascade's three-tier bound (wgs) or
// the plain decode's one-tier bound, whichever is larger.
static int decode_num_ranges(int num_seqs, int max_context_len, int num_kv_heads, int (&wgs)[kTiers]) {
  decode_schedule(num_seqs, max_context_len, num_kv_heads, wgs);
  int tiers = 0;
  for (int t = 0; t < kTiers; ++t) tiers += wgs[t];
  const int64_t umax = static_cast<int64_t>(num_kv_heads) * num_seqs *
                       ((static_cast<int64_t>(max_context_len) + kBlk - 1) / kBlk);
  const int64_t n = std::min<int64_t>(kPlainRanges, (umax + kOneTierMin - 1) / kOneTierMin);
  const int one = static_cast<int>(n < 1 ? 1 : n) + (kTiers - 1);
  return std::max(tiers, one);
}

DecodePlan plan_decode(int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, int dtype, int cache_fp8) {
  (void)cache_fp8;                    // both cache formats have the stream kernel
  DecodePlan p{};
  const int G = num_heads / num_kv_heads;
  p.fast = dtype == kBF16 && head_dim == kD &&
           (block_size == kBlk || block_size == 2 * kBlk || block_size == 4 * kBlk) && G >= 1 &&
           G <= kMaxG;
  if (!p.fast) return p;
  int wgs[kTiers];
  p.num_ranges = decode_num_ranges(num_seqs, max_context_len, num_kv_heads, wgs);
  p.ws_bytes = kWsHeader + arrive_bytes(p.num_ranges) +
               static_cast<size_t>(2) * p.num_ranges * G * (kD + 2) * sizeof(float);
  return p;
}

// log2 of the cache block size in 16-token blocks (16, 32, 64 tokens; validated on the host)
static int block_shift(int block_size) { return block_size == 4 * kBlk ? 2 : block_size == 2 * kBlk ? 1 : 0; }

template <int G, int BS>
static void launch_stream_bs(const DecodeKArgs& k, const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.cache_fp8)
    hipLaunchKernelGGL((decode_stream_kernel<G, true, false, BS>), dim3(grid), dim3(kThreads), 0,
                       stream, k);
  else
    hipLaunchKernelGGL((decode_stream_kernel<G, false, false, BS>), dim3(grid), dim3(kThreads), 0,
                       stream, k);
}

template <int G>
static void launch_stream(const DecodeKArgs& k, const AttnArgs& a, hipStream_t stream) {
  // up to two workgroups per CU; those past the batch's R leave at once
  const int grid = k.num_ranges < kPlainRanges ? k.num_ranges : kPlainRanges;
  hipLaunchKernelGGL(decode_claim_reset_kernel, dim3(1), dim3(256), 0, stream, k.claim, k.arrive,
                     k.num_ranges);
  switch (block_shift(a.block_size)) {
    case 0: launch_stream_bs<G, 0>(k, a, grid, stream); break;
    case 1: launch_stream_bs<G, 1>(k, a, grid, stream); break;
    default: launch_stream_bs<G, 2>(k, a, grid, stream); break;
  }
}

static DecodeKArgs make_kargs(const AttnArgs& a) {
  DecodeKArgs k{};
  const int G = a.num_heads / a.num_kv_heads;
  k.q = static_cast<const uint16_t*>(a.q);
  k.q_stride = a.q_stride;
  k.k_cache = static_cast<const uint8_t*>(a.k_cache);
  k.v_cache = static_cast<const uint8_t*>(a.v_cache);
  k.num_blocks = a.num_blocks;
  k.block_tables = a.block_tables;
  k.max_blocks = a.max_blocks;
  k.context_lens = a.context_lens;
  k.num_seqs = a.num_seqs;
  k.out = static_cast<uint16_t*>(a.out);
  k.out_stride = a.out_stride;
  k.num_heads = a.num_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.max_context_len = a.max_context_len;
  k.num_ranges = decode_num_ranges(a.num_seqs, a.max_context_len, a.num_kv_heads, k.tier_wgs);
  k.scale_log2 = a.scale * kLog2e * (a.cache_fp8 ? a.k_scale : 1.0f);
  k.out_scale = a.cache_fp8 ? a.v_scale : 1.0f;
  k.err = a.err;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  k.claim = reinterpret_cast<int*>(ws);
  k.arrive = reinterpret_cast<int*>(ws + kWsHeader);
  k.ws_acc = reinterpret_cast<float*>(ws + kWsHeader + arrive_bytes(k.num_ranges));
  k.ws_ml = k.ws_acc + static_cast<size_t>(2) * k.num_ranges * G * kD;
  return k;
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (!p.fast) return launch_attn_generic(a, stream);
  const int G = a.num_heads / a.num_kv_heads;
  const DecodeKArgs k = make_kargs(a);
  switch (G) {
    case 1: launch_stream<1>(k, a, stream); break;
    case 2: launch_stream<2>(k, a, stream); break;
    case 3: launch_stream<3>(k, a, stream); break;
    case 4: launch_stream<4>(k, a, stream); break;
    case 5: launch_stream<5>(k, a, stream); break;
    case 6: launch_stream<6>(k, a, stream); break;
    case 7: launch_stream<7>(k, a, stream); break;
    default: launch_stream<8>(k, a, stream); break;
  }
  return hipGetLastError();
}

// ---- cascade plan and launch ----
static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

CascadePlan plan_cascade(int num_seqs, int max_context_len, int max_prefix_len, int num_members,
                         int num_prefixes, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int dtype, int cache_fp8) {
  CascadePlan c{};
  c.dec = plan_decode(num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                      dtype, cache_fp8);
  c.ws_bytes = c.dec.ws_bytes;
  if (!c.dec.fast) return c;
  // prefixes are whole cache blocks; chunks count 16-token blocks
  const int max_pb = max_prefix_len / block_size * (block_size / kBlk);
  c.active = max_pb > 0 && num_members > 0 && num_prefixes > 0;
  if (!c.active) return c;
  const int G = num_heads / num_kv_heads;
  int cb = (max_pb + 15) / 16;            // about 16 chunks of 8..64 blocks
  cb = cb < 8 ? 8 : (cb > 64 ? 64 : cb);
  c.chunk_blocks = cb;
  c.max_chunks = (max_pb + cb - 1) / cb;
  c.col_wgs = static_cast<int>((static_cast<int64_t>(num_members) * G + 16 * kNW - 1) / (16 * kNW));
  c.tasks = static_cast<int64_t>(c.col_wgs) * num_prefixes * num_kv_heads * c.max_chunks;
  const size_t rows = static_cast<size_t>(c.max_chunks) * num_seqs * num_heads;
  c.cas_off = round256(c.dec.ws_bytes);
  c.pre_ml_off = c.cas_off + round256(static_cast<size_t>(num_seqs) * sizeof(int2));
  c.pre_acc_off = c.pre_ml_off + round256(rows * 2 * sizeof(float));
  c.ws_bytes = c.pre_acc_off + rows * kD * sizeof(float);
  return c;
}

template <int G, int BS>
static void launch_cascade_bs(const DecodeKArgs& k, const CascadeArgs& ca, int grid, dim3 pgrid,
                              const AttnArgs& a, hipStream_t stream) {
  if (a.cache_fp8) {
    hipLaunchKernelGGL((decode_prefix_kernel<G, true, BS>), pgrid, dim3(kThreads), 0, stream, k, ca);
    hipLaunchKernelGGL((decode_stream_kernel<G, true, true, BS>), dim3(grid), dim3(kThreads), 0,
                       stream, k);
  } else {
    hipLaunchKernelGGL((decode_prefix_kernel<G, false, BS>), pgrid, dim3(kThreads), 0, stream, k, ca);
    hipLaunchKernelGGL((decode_stream_kernel<G, false, true, BS>), dim3(grid), dim3(kThreads), 0,
                       stream, k);
  }
}

template <int G>
static void launch_cascade_g(const DecodeKArgs& k, const CascadeArgs& ca, int64_t tasks,
                             const AttnArgs& a, hipStream_t stream) {
  const int grid = k.num_ranges < kCUs ? k.num_ranges : kCUs;
  const dim3 pgrid(static_cast<unsigned>(1 + tasks));
  switch (block_shift(a.block_size)) {
    case 0: launch_cascade_bs<G, 0>(k, ca, grid, pgrid, a, stream); break;
    case 1: launch_cascade_bs<G, 1>(k, ca, grid, pgrid, a, stream); break;
    default: launch_cascade_bs<G, 2>(k, ca, grid, pgrid, a, stream); break;
  }
}

hipError_t launch_decode_cascade(const AttnArgs& a, const CascadeMeta& m, const CascadePlan& p,
                                 hipStream_t stream) {
  if (!p.active) return launch_decode(a, p.dec, stream);
  const int G = a.num_heads / a.num_kv_heads;
  DecodeKArgs k = make_kargs(a);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  k.cas = reinterpret_cast<int2*>(ws + p.cas_off);
  k.pre_ml = reinterpret_cast<float*>(ws + p.pre_ml_off);
  k.pre_acc = reinterpret_cast<float*>(ws + p.pre_acc_off);
  CascadeArgs ca{};
  ca.indptr = m.indptr;
  ca.seqs = m.seqs;
  ca.lens = m.lens;
  ca.num_prefixes = m.num_prefixes;
  ca.num_members = m.num_members;
  ca.max_prefix_len = m.max_prefix_len;
  ca.chunk_blocks = p.chunk_blocks;
  ca.max_chunks = p.max_chunks;
  ca.col_wgs = p.col_wgs;
  switch (G) {
    case 1: launch_cascade_g<1>(k, ca, p.tasks, a, stream); break;
    case 2: launch_cascade_g<2>(k, ca, p.tasks, a, stream); break;
    case 3: launch_cascade_g<3>(k, ca, p.tasks, a, stream); break;
    case 4: launch_cascade_g<4>(k, ca, p.tasks, a, stream); break;
    case 5: launch_cascade_g<5>(k, ca, p.tasks, a, stream); break;
    case 6: launch_cascade_g<6>(k, ca, p.tasks, a, stream); break;
    case 7: launch_cascade_g<7>(k, ca, p.tasks, a, stream); break;
    default: launch_cascade_g<8>(k, ca, p.tasks, a, stream); break;
  }
  return hipGetLastError();
}

}  // namespace qw
