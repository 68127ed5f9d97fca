// Varlen causal GQA prefill over the paged cache on gfx950 matrix cores.
//
// What is computed: for each sequence s with n new rows and context c, row i
// (position c - n + i) of query head h attends to keys 0 .. c - n + i of KV
// head h / G ("Qwen2大模型架构解析与vLLM优化实践", §7.3 causal mask; "Qwen 开源
// 工程笔记", §3 packed varlen prefill; "Qwen2 模型结构代码详解", §2 GQA and
// scaling head_dim^-0.5), keys gathered through the block table ("vLLM 部署
// Qwen", §2.1).
//
// bf16, head_dim 128, cache blocks of 16, 32 or 64 tokens (keys are taken
// in 16-token blocks), group G <= 8:
//   * one workgroup per (KV head, query tile, sequence), in one of two
//     layouts chosen per launch by a cost estimate (key_groups below):
//     - one key group: G waves, a wave owns 32 query columns = one head of
//       the group x 32 rows, keys in steps of 32;
//     - two key groups: a wave owns 32 columns = 2 heads x 16 rows (an odd
//       group pads its last wave with a copy of the last head, whose output
//       is dropped); the workgroup holds two sets of ceil(G/2) waves, and
//       keys stream in steps of 64 (four cache blocks) of which key group k
//       takes keys 32k .. 32k + 31.  The two groups' online-softmax states
//       are merged through LDS at the end, so a query tile's keys are
//       covered in half the steps (short tiles, long contexts);
//   * steps (16 or 32 KiB of K and V^T) go through a ring of four LDS stages
//     with direct-to-LDS buffer loads (no register staging), processed in
//     pairs: one load wait and one barrier per two steps, the next pair's
//     loads in flight meanwhile.  With at least 4 KG waves each of the first
//     4 KG waves issues the four 1 KiB loads of one (tile, K or V, block)
//     group through one descriptor (the CU's scalar unit is shared: 16 KG
//     separately built loads per step kept it busy); with fewer waves each
//     wave issues the same number of loads (surplus ones have an empty range
//     and land in a scratch line).  Either way a wave's outstanding-load
//     count at every wait is a compile-time constant;
//   * the block ids the workgroup needs are staged in LDS once (the first 64
//     also in a register of every wave, read with v_readlane), so no load
//     inside the loop depends on another load.  Their LDS is sized per
//     launch from the longest context beside the stages: up to ~120K-token
//     contexts with two key groups, ~380K with one (which takes the longer
//     ones);
//   * LDS layouts are XOR-swizzled at 16-byte granularity (the source address
//     of each loaded chunk is chosen so that it lands in its swizzled slot):
//     every 16-lane group of an MFMA operand read hits 16 distinct bank groups;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//     B = the wave's Q^T held in registers), so each lane owns one query
//     column: the softmax max and sum over keys are in-lane plus one
//     exchange between the two lane halves;
//   * online softmax in base 2 (scores scaled by scale * log2 e inside the
//     exponent); the running max is raised only when a column's tile max
//     exceeds it by more than 8 (probabilities stay below 2^8, exact in bf16
//     range and harmless to the fp32 sums), so the output rescale is rare;
//   * O^T += V^T P^T with the same MFMA: P^T comes straight from the S^T
//     accumulator registers (rounded to bf16), V^T is read from LDS.  The K
//     rows feeding the MFMA are permuted (bits 2 and 3 of the key index
//     swapped) so that the keys each lane holds in P^T are 8 consecutive
//     keys, which the dims-major V cache tile stores contiguously;
//   * key tiles past the causal limit of the query tile are skipped; the
//     grid is issued longest tile level first, XCD- and shader-engine-aware
//     (see the work-item mapping at the top of the kernel).
// FP8 caches: the same kernel with the codes widened to bf16 on their way
// into LDS (the F8 variant).  Other shapes and fp32 use the generic kernel.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace qw {

namespace {

constexpr int kD = 128;
constexpr int kB = 16;               // tokens per key block (a cache block holds 16, 32 or 64)
constexpr int kBK = 32;              // keys per key group and step
constexpr int kTile = 16384;         // bytes of one 32-key tile in LDS: K 8 KiB + V^T 8 KiB
constexpr int kTileLoads = 16;       // 1 KiB direct-to-LDS loads per 32-key tile
constexpr int kBlockBytes = kB * kD * 2;   // one head's K of one 16-token key block
constexpr int kLdsBytes = 160 * 1024;   // LDS of one CU (a workgroup's static + dynamic share)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;        // raise the running max only past this margin (log2 units)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PrefillKArgs {
  const uint16_t* q; int64_t q_stride;
  const uint16_t* k_cache; const uint16_t* v_cache; int num_blocks;
  const int32_t* cu_seqlens; const int32_t* context_lens;
  const int32_t* block_tables; int max_blocks;
  uint16_t* out; int64_t out_stride;
  int num_tokens, max_context_len, num_heads, num_kv_heads;
  int num_seqs, num_qtiles, pairs_per_xcd;        // pairs_per_xcd 0: plain order
  float scale_log2;                               // scale * log2 e (* k_scale for an FP8 cache)
  float out_scale;                                // 1, or v_scale for an FP8 cache
  unsigned* err;                                  // the device error word (may be null)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// max of x over lanes i and i ^ 32, in registers (v_permlane32_swap swaps
// the two halves of its operands; whichever result holds the other half,
// the max of x and both results is the pair's max)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
// swap bits 2 and 3 of a 4-bit index (its own inverse)
__device__ __forceinline__ int perm23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
// V^T slot swizzle bit of dims row d
__device__ __forceinline__ int vswz(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

// key held by accumulator register r of a lane in half h (see the K row
// permutation above): 8 consecutive keys per 16-key chunk
__device__ __forceinline__ int key_of(int r, int h) { return (r & 7) + 8 * h + 16 * (r >> 3); }

// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// workgroup barrier without the release/acquire fences of __syncthreads: the
// fences would wait for every outstanding direct-to-LDS load.  Callers wait
// for what must be complete first; the memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16 bytes per lane from buffer rs at byte offset voff into LDS at lds + 16 * lane
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// LDS layout of one 32-key tile (16-byte slots):
//   K tile: slot(R, c) = R * 16 + (c ^ perm23(R & 15)), key R of the tile
//           (0..31), dims chunk c (8 dims, 0..15);
//   V^T tile (bytes 8192..): slot(b, d, h) = b * 256 + d * 2 + (h ^ vswz(d)),
//           cache block b of the tile, dims row d, 8-key half h.
// Load j (0..15) of a tile fills slots 64 j .. 64 j + 63: loads 0..7 the K
// tile (block j / 4), loads 8..15 the V^T tile (block (j - 8) / 4).  Byte
// offset inside the head's 16-token (sub-)block of the chunk lane `lane`
// fetches (vrow: bytes of one dims row of the V cache tile):
__device__ __forceinline__ int load_offset(int j, int lane, int vrow) {
  if (j < 8) {
    const int kk = 4 * (j & 3) + (lane >> 4);          // key within the cache block
    const int c = (lane & 15) ^ perm23(kk);
    return kk * (kD * 2) + c * 16;
  }
  const int u = ((j - 8) & 3) * 64 + lane;
  const int d = u >> 1;
  const int h = (u & 1) ^ vswz(d);
  return d * vrow + h * 16;
}

// two E4M3FN codes (bytes 2 HI, 2 HI + 1 of w) -> a bf16 pair, exactly
// (every E4M3FN value is a bf16 value)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// KG key groups (1 or 2) of WPG waves each.  A wave owns 32 query columns:
// one head x 32 rows (KG 1) or two heads x 16 rows (KG 2).
// F8: the caches hold E4M3FN codes.  Their tiles (half the bytes) are read
// into registers, widened exactly to bf16 and written to the same LDS
// layout, one step ahead of the arithmetic; k_scale is folded into the
// score scale and v_scale into the output.
// BS: cache blocks of 16 << BS tokens, read as 16-token blocks.
template <int KG, int WPG, bool F8, int BS>
__global__ __launch_bounds__(KG * WPG * 64) void prefill_mfma_kernel(PrefillKArgs a) {
  constexpr int NW = KG * WPG;                    // waves
  constexpr int HPW = KG == 1 ? 1 : 2;            // heads per wave
  constexpr int kBQ = 32 / HPW;                   // query rows per tile
  constexpr int kStage = KG * kTile;              // one step's keys (32 KG)
  constexpr int kLoads = KG * kTileLoads;         // loads per step
  // With at least 4 KG waves, wave w < 4 KG issues the four 1 KiB loads of
  // one whole (tile, K or V, cache block) group through one descriptor and
  // the other waves issue none: every descriptor and LDS address is built
  // once per step by one wave (the scalar unit is shared by the CU's waves,
  // and 16 KG separately built loads kept it busy for hundreds of cycles
  // per step).  Fewer waves take loads j = wave + NW i.
  constexpr bool GROUPED = NW >= 4 * KG;
  constexpr int NI = GROUPED ? 4 : (kLoads + NW - 1) / NW;   // loads per loading wave per step
  // work item of this workgroup: (KV head g, sequence s, query tile qt)
  const int np = a.num_kv_heads * a.num_seqs;     // (g, s) pairs
  int p, z;
  if (a.pairs_per_xcd > 0) {
    // workgroup L runs on XCD L % 8; pair p lives on XCD p % 8 so its K/V
    // stay in one L2.  Within an XCD, consecutive workgroups go round-robin
    // to its shader engines: rotating the pair order by the tile level
    // spreads each pair's tiles over all of them.
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    z = j / a.pairs_per_xcd;
    p = x + 8 * ((j + z) % a.pairs_per_xcd);
    if (p >= np) return;
  } else {
    z = blockIdx.x / np;
    p = blockIdx.x % np;
  }
  const int G = a.num_heads / a.num_kv_heads;
  const int g = p % a.num_kv_heads, s = p / a.num_kv_heads;
  const int qt = a.num_qtiles - 1 - z;            // longest (last) tiles first
  const int tid = threadIdx.x;
  // this thread's block-table entry, fetched before (and in parallel with)
  // the sequence metadata: the table row needs only s
  const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  constexpr int bsh = BS;
  const int bt_early = (tid >> bsh) < a.max_blocks ? bt[tid >> bsh] : 0;
  // the first 64 block ids again, lane i of every wave holding block i: the
  // first steps take their ids with v_readlane instead of an LDS round trip
  const int lane_id = tid & 63;
  int idv = (lane_id >> bsh) < a.max_blocks ? bt[lane_id >> bsh] : 0;
  // the sequence's context length is fetched with its row range, not after
  // it (one memory latency less before the first tile loads)
  int ctx = a.context_lens[s];
  const int r0 = a.cu_seqlens[s];
  const int r1 = a.cu_seqlens[s + 1];
  asm volatile("" ::"s"(ctx), "s"(r0), "s"(r1));  // all three loaded here (none sunk past the exit)
  const int n = r1 - r0;
  const int q0 = qt * kBQ;
  if (q0 >= n) {
    if (n < 0 && qt == 0 && tid == 0) report_error(a.err, kErrSequence);
    return;
  }
  // rows outside the packed batch, or more rows than any valid context
  // holds (the block-id staging is sized for max_context_len keys): flag,
  // write nothing
  const bool rows_bad = r0 < 0 || r0 + n > a.num_tokens || n > a.max_context_len;
  bool bad = rows_bad || ctx < n || ctx > a.max_context_len;
  if (bad && tid == 0) report_error(a.err, kErrSequence);
  if (rows_bad) return;
  if (bad) ctx = n;                               // keep every index in range; output is NaN
  const int pos0 = ctx - n;                       // position of row 0
  const int qlast = min(q0 + kBQ, n) - 1;         // last valid row of the tile
  const int nkt = (pos0 + qlast) / kBK + 1;       // 32-key tiles up to the causal limit
  const int nst = (nkt + KG - 1) / KG;            // steps (KG tiles each)
  const int nblk = (ctx + kB - 1) / kB;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int kg = wave / WPG;                      // key group
  const int hw = wave - kg * WPG;                 // wave within the group
  const int hl = lane >> 5;                       // lane half
  const int col = lane & 31;                      // query column of this lane
  const int hslot = HPW * hw + col / kBQ;         // head of the group for this column
  const int hq = g * G + min(hslot, G - 1);       // query head (padding column: a copy)
  const int rq = col % kBQ;                       // row within the tile

  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t trash[1024];
  __shared__ int sbad;
  // block ids of steps 0 .. nst - 1, sized per launch for the longest context
  extern __shared__ __attribute__((aligned(16))) int sids[];

  // Q^T operand: column = (head, row q0 + rq (clamped)), 8 dims per k-step
  bf16x8_t qb[kD / 16];
  {
    const int row = min(q0 + rq, n - 1);
    const uint16_t* qp = a.q + static_cast<int64_t>(r0 + row) * a.q_stride +
                         static_cast<int64_t>(hq) * kD + hl * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 16));
  }

  // stage the block ids; ids past the context or out of the pool read block
  // 0.  The barrier waits for the table loads only: the Q loads (issued
  // later) stay in flight until the first tile's wait.
  {
    bool lbad = false;
    for (int i = tid; i < 2 * KG * nst; i += NW * 64) {
      int blk = 0;
      if (i < nblk) {
        blk = i == tid ? bt_early : bt[i >> bsh];
        if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
          lbad = true;
          blk = 0;
        }
      }
      sids[i] = blk;
    }
    if (tid == 0) sbad = 0;
    wait_lds();
    barrier();
    if (lbad) sbad = 1;
    if (lane_id >= nblk || static_cast<unsigned>(idv) >= static_cast<unsigned>(a.num_blocks)) idv = 0;
  }

  // per-lane source offsets of this wave's loads (grouped: load i of group
  // wave is j = 4 (wave % 4) + i of tile wave / 4; otherwise load j = wave +
  // NW i, j / 16 the 32-key tile of the step, j % 16 the load within it)
  // (kept in registers when there are few; recomputed per load otherwise)
  const bool loader = !GROUPED || wave < 4 * KG;  // wave-uniform
  const int vrow = (kB * 2) << bsh;               // bytes of a V cache tile's dims row
  constexpr int NV = NI <= 8 ? NI : 1;
  int voff[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = GROUPED ? 16 * (wave >> 2) + 4 * (wave & 3) + i : wave + NW * i;
    voff[i] = loader && j < kLoads ? load_offset(j & 15, lane, vrow) : 0;
  }
  const int64_t head_off = static_cast<int64_t>(g) * (kB * kD << bsh);
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * (kB * kD << bsh);
  const int submask = (1 << bsh) - 1;
  const int vrange = (127 * (kB << bsh) + kB) * 2;   // V bytes from a sub-block's start

  // issue the loads of step t's keys into stage dst; a 32-key tile past the
  // causal limit gets empty ranges (no traffic).  Forced inline: with one or
  // two waves a wave issues 16 loads per step, and the compiler would
  // otherwise make this a real call inside the step loop.
  auto issue = [&](int t, uint8_t* dst) __attribute__((always_inline)) {
    int b0, b1, b2 = 0, b3 = 0;                   // block ids of the step
    if (2 * KG * t + 2 * KG <= 64) {              // from the register (uniform branch)
      b0 = __builtin_amdgcn_readlane(idv, 2 * KG * t);
      b1 = __builtin_amdgcn_readlane(idv, 2 * KG * t + 1);
      if constexpr (KG == 2) {
        b2 = __builtin_amdgcn_readlane(idv, 4 * t + 2);
        b3 = __builtin_amdgcn_readlane(idv, 4 * t + 3);
      }
    } else if constexpr (KG == 2) {
      const int4 ids = *reinterpret_cast<const int4*>(&sids[4 * t]);
      b0 = uniform(ids.x), b1 = uniform(ids.y), b2 = uniform(ids.z), b3 = uniform(ids.w);
    } else {
      const int2 ids = *reinterpret_cast<const int2*>(&sids[2 * t]);
      b0 = uniform(ids.x), b1 = uniform(ids.y);
    }
    if constexpr (GROUPED) {
      if (!loader) return;
      const int half = wave >> 2, jj0 = 4 * (wave & 3);   // this wave's group
      const int bi = 2 * half + ((jj0 >> 2) & 1);
      const int blk = bi == 0 ? b0 : bi == 1 ? b1 : bi == 2 ? b2 : b3;
      const bool live = KG * t + half < nkt;
      const int sub = (2 * KG * t + bi) & submask;   // 16-token sub-block of the entry
      const bool isv = jj0 >= 8;
      const uint16_t* base = (isv ? a.v_cache : a.k_cache) + blk * blk_elems + head_off +
                             sub * (isv ? kB : kB * kD);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base), static_cast<short>(0),
          live ? (isv ? vrange : kBlockBytes) : 0, 0x00020000);
      uint8_t* d = dst + half * kTile + jj0 * 1024;
#pragma unroll
      for (int i = 0; i < 4; ++i) load_lds16(rs, d + i * 1024, voff[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = wave + NW * i;
      const int half = KG == 2 ? (j >> 4) & 1 : 0, jj = j & 15;
      const bool live = j < kLoads && KG * t + half < nkt;
      const int bi = 2 * half + ((jj >> 2) & 1);
      const int blk = bi == 0 ? b0 : bi == 1 ? b1 : bi == 2 ? b2 : b3;
      const int sub = (2 * KG * t + bi) & submask;
      const bool isv = jj >= 8;
      const uint16_t* base = (isv ? a.v_cache : a.k_cache) + blk * blk_elems + head_off +
                             sub * (isv ? kB : kB * kD);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base), static_cast<short>(0),
          live ? (isv ? vrange : kBlockBytes) : 0, 0x00020000);
      const int vo = NI <= 8 ? voff[i < NV ? i : 0] : (j < kLoads ? load_offset(jj, lane, vrow) : 0);
      load_lds16(rs, j < kLoads ? dst + half * kTile + jj * 1024 : trash, vo);
    }
  };

  // V^T entries of keys >= ctx may hold anything (NaN): zero them, a zero
  // probability times NaN would poison the row
  auto sanitize = [&](int t, uint8_t* stg) {
    for (int sl = tid; sl < KG * 512; sl += NW * 64) {
      const int half = sl >> 9, w = sl & 511;
      const int b = w >> 8, u = w & 255, d = u >> 1;
      const int h = (u & 1) ^ vswz(d);
      const int key0 = t * KG * kBK + half * kBK + b * kB + h * 8;
      if (key0 + 8 > ctx) {
        uint4* vt = reinterpret_cast<uint4*>(stg + half * kTile + 8192) + w;
        uint4 v = *vt;
        uint32_t* e = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k0 = key0 + 2 * q;
          uint32_t x = e[q];
          if (k0 >= ctx) x &= 0xffff0000u;
          if (k0 + 1 >= ctx) x &= 0x0000ffffu;
          e[q] = x;
        }
        *vt = v;
      }
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  // running max (log2 units) and sum.  The max starts at the most negative
  // finite float, not -inf: a column whose keys in a key group's first tile
  // are all masked then gets probabilities exp2(-inf) = 0 there instead of
  // exp2(-inf + inf) = NaN (with two key groups the second group's first
  // tile can lie wholly past a row).  Its first visible tile raises the max
  // and scales the (zero) state by exp2(-FLT_MAX - max) = 0 as -inf did.
  float m = -__FLT_MAX__, l = 0.0f;
  const int qpos = pos0 + q0 + rq;
  const float c2 = a.scale_log2;

  // K row read by this lane for the S^T MFMA: MFMA row i = col holds key
  // perm23(i) of the tile; its dims chunk c sits in slot c ^ (col & 15)
  const int krow = (col & 16) | perm23(col & 15);
  const int kx = hl ^ (col & 15);
  const int vlane = (col * 2 + (hl ^ vswz(col))) * 16;
  const int sani_st = (ctx % (KG * kBK)) ? ctx / (KG * kBK) : -1;   // step holding keys >= ctx
  const int tile_off = kg * kTile;                // this key group's tile in a stage

  // S^T = K Q^T of this group's tile in stage stg
  auto qk = [&](const uint8_t* stg) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint8_t* kp = stg + tile_off + krow * (kD * 2);
#pragma unroll
    for (int kb = 0; kb < kD / 16; kb += 4) {     // K fragments four at a time (register pressure)
      bf16x8_t ka[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ka[i] = as_bf16x8(*reinterpret_cast<const uint4*>(kp + ((2 * (kb + i)) ^ kx) * 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qb[kb + i], acc, 0, 0, 0);
    }
    return acc;
  };

  // causal mask of a diagonal 32-key tile kt (some key lies past some row)
  auto mask = [&](int kt, f32x16_t& sc) {
    if (kt * kBK + kBK - 1 > pos0 + q0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = (kt * kBK + key_of(r, hl) <= qpos) ? sc[r] : -INFINITY;
    }
  };

  // online softmax of a masked score tile (base 2): new running max, sum and
  // the bf16 probabilities.  Returns the factor the output must be scaled by
  // (1 for columns whose max stays).
  bf16x8_t pb[2];
  auto softmax = [&](const f32x16_t& sc) {
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = max_halves(mt) * c2;
    // each column decides from its own scores alone (a column's result must
    // not depend on its neighbours)
    const bool up = mt > m + kLazy;
    const float alpha = up ? __builtin_amdgcn_exp2f(m - mt) : 1.0f;
    m = up ? mt : m;
    float lt = 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c * 8 + j], c2, -m));
        lt += pr;
        pb[c][j] = static_cast<__bf16>(pr);
      }
    }
    l = l * alpha + lt;
    return alpha;
  };

  // O^T = alpha O^T + V^T P^T for this group's tile in stage stg
  auto pv = [&](float alpha, const uint8_t* stg) {
    const uint8_t* vp = stg + tile_off + 8192 + vlane;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {                 // V fragments per 16-key half (register pressure)
      bf16x8_t va[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        va[dt] = as_bf16x8(*reinterpret_cast<const uint4*>(vp + c * 4096 + dt * 1024));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], pb[c], o[dt], 0, 0, 0);
    }
  };

  // softmax and PV of a score tile of 32-key tile kt held in stage stg
  auto finish = [&](int kt, f32x16_t sc, const uint8_t* stg) {
    mask(kt, sc);
    const float alpha = softmax(sc);
    pv(alpha, stg);
  };

  if constexpr (F8) {
    // Chunk i of a step (8 codes -> one 16-byte LDS slot), tile hf = i / 1024
    // of the step, w = i % 1024:
    //   w < 512:  key R = w / 16 of the tile, dims chunk c = w % 16: codes at
    //             (R % 16) * 128 + 8 c of block R / 16's K tile ([B][d]),
    //             K slot R * 16 + (c ^ perm23(R % 16));
    //   w >= 512: v = w - 512, block b = v / 256, dims row d = (v % 256) / 2,
    //             keys 8 h .. 8 h + 7 (h = v % 2): codes at d * 16 + 8 h of the
    //             V tile ([d][B]), V^T slot 512 + b * 256 + d * 2 + (h ^ vswz(d)).
    // V entries of keys >= ctx are written as zeros (slots there may hold
    // anything, a zero probability times NaN would poison the row).
    constexpr int kChunks = KG * 1024;
    constexpr int NCH = (kChunks + NW * 64 - 1) / (NW * 64);
    constexpr int kTile8 = kB * kD;                 // bytes of one head's FP8 K (or V) block tile
    const uint8_t* kc8 = reinterpret_cast<const uint8_t*>(a.k_cache);
    const uint8_t* vc8 = reinterpret_cast<const uint8_t*>(a.v_cache);
    const int64_t head8 = static_cast<int64_t>(g) * (kTile8 << bsh);
    const int64_t blk8 = static_cast<int64_t>(a.num_kv_heads) * (kTile8 << bsh);
    auto gload = [&](int t, uint2 (&r)[NCH]) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = tid + i * NW * 64;
        r[i] = make_uint2(0u, 0u);
        if (ci < kChunks) {
          const int hf = ci >> 10, w = ci & 1023;
          int b, off;
          const uint8_t* base;
          if (w < 512) {
            const int R = w >> 4;
            b = R >> 4;
            off = (R & 15) * kD + (w & 15) * 8;
            base = kc8;
          } else {
            const int v = w - 512;
            b = v >> 8;
            off = ((v & 255) >> 1) * (kB << bsh) + (v & 1) * 8;
            base = vc8;
          }
          const int u = 2 * (KG * t + hf) + b;      // 16-token block of the sequence
          off += (u & submask) * (w < 512 ? kB * kD : kB);
          const int blk = sids[u];
          r[i] = *reinterpret_cast<const uint2*>(base + blk * blk8 + head8 + off);
        }
      }
    };
    auto commit = [&](int t, const uint2 (&r)[NCH], uint8_t* dst) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = tid + i * NW * 64;
        if (ci < kChunks) {
          const int hf = ci >> 10, w = ci & 1023;
          uint4 x = make_uint4(fp8x2_bf16x2<false>(r[i].x), fp8x2_bf16x2<true>(r[i].x),
                               fp8x2_bf16x2<false>(r[i].y), fp8x2_bf16x2<true>(r[i].y));
          int slot;
          if (w < 512) {
            const int R = w >> 4;
            slot = R * 16 + ((w & 15) ^ perm23(R & 15));
          } else {
            const int v = w - 512;
            const int b = v >> 8, d = (v & 255) >> 1, h = v & 1;
            slot = 512 + b * 256 + d * 2 + (h ^ vswz(d));
            const int key0 = t * KG * kBK + hf * kBK + b * kB + h * 8;
            if (key0 + 8 > ctx) {
              uint32_t* e = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int k0 = key0 + 2 * q;
                uint32_t y = e[q];
                if (k0 >= ctx) y &= 0xffff0000u;
                if (k0 + 1 >= ctx) y &= 0x0000ffffu;
                e[q] = y;
              }
            }
          }
          *reinterpret_cast<uint4*>(dst + hf * kTile + slot * 16) = x;
        }
      }
    };
    // registers: step s in ra (s even) or rb (s odd), two steps in flight;
    // LDS: step s in st0 (s even) or st1 (s odd).  Step t: the arithmetic of
    // step t, then step t + 1 widened into the other stage (every wave passed
    // the barrier after step t - 1, so that stage is free), then step t + 3's
    // loads into the registers step t + 1 freed; one barrier.
    uint2 ra[NCH], rb[NCH];
    gload(0, ra);
    if (nst > 1) gload(1, rb);
    commit(0, ra, st0);
    if (nst > 2) gload(2, ra);
    wait_lds();
    barrier();
    for (int t = 0; t < nst; t += 2) {
      if (KG * t + kg < nkt) finish(KG * t + kg, qk(st0), st0);
      if (t + 1 < nst) {
        commit(t + 1, rb, st1);
        if (t + 3 < nst) gload(t + 3, rb);
      }
      wait_lds();
      barrier();
      if (t + 1 >= nst) break;
      if (KG * (t + 1) + kg < nkt) finish(KG * (t + 1) + kg, qk(st1), st1);
      if (t + 2 < nst) {
        commit(t + 2, ra, st0);
        if (t + 4 < nst) gload(t + 4, ra);
      }
      wait_lds();
      barrier();
    }
  } else {
  // Steps in pairs: one wait and one barrier for two steps (the pair's
  // keys, loaded during the previous pair), then the next pair's loads into
  // the two stages the previous pair used, then both steps' arithmetic with
  // no barrier between them.
  auto pair = [&](int t, uint8_t* c0, uint8_t* c1, uint8_t* r0, uint8_t* r1)
      __attribute__((always_inline)) {
    if (loader) wait_vm<0>();
    barrier();
    if (t == sani_st || t + 1 == sani_st) {
      sanitize(sani_st, t == sani_st ? c0 : c1);
      wait_lds();
      barrier();
    }
    if (t + 2 < nst) issue(t + 2, r0);
    if (t + 3 < nst) issue(t + 3, r1);
    if (KG * t + kg < nkt) finish(KG * t + kg, qk(c0), c0);
    if (t + 1 < nst && KG * (t + 1) + kg < nkt) finish(KG * (t + 1) + kg, qk(c1), c1);
  };
  issue(0, st0);
  if (nst > 1) issue(1, st1);
  for (int t = 0; t < nst; t += 4) {
    pair(t, st0, st1, st2, st3);
    if (t + 2 >= nst) break;
    pair(t + 2, st2, st3, st0, st1);
  }
  }

  __syncthreads();
  if (sbad) {
    bad = true;
    if (tid == 0) report_error(a.err, kErrBlock);
  }
  uint8_t* mg = hw == 0 ? st0 : hw == 1 ? st1 : hw == 2 ? st2 : st3;
  if constexpr (KG == 2) {
  // ---- merge the key groups through LDS (the ring is free now) ----
  float4* mo = reinterpret_cast<float4*>(mg);
  float* ml = reinterpret_cast<float*>(mg + 16 * 64 * 16);
  if (kg == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        mo[(dt * 4 + r4) * 64 + lane] = make_float4(o[dt][r4 * 4], o[dt][r4 * 4 + 1],
                                                    o[dt][r4 * 4 + 2], o[dt][r4 * 4 + 3]);
    ml[lane] = m;
    ml[64 + lane] = l;
  }
  __syncthreads();
  if (kg == 1) return;
  {
    const float m1 = ml[lane], l1 = ml[64 + lane];
    const float mm = fmaxf(m, m1);
    const float a0 = __builtin_amdgcn_exp2f(m - mm);
    const float a1 = __builtin_amdgcn_exp2f(m1 - mm);   // 0 when group 1 saw no key
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 v = mo[(dt * 4 + r4) * 64 + lane];
        o[dt][r4 * 4 + 0] = o[dt][r4 * 4 + 0] * a0 + v.x * a1;
        o[dt][r4 * 4 + 1] = o[dt][r4 * 4 + 1] * a0 + v.y * a1;
        o[dt][r4 * 4 + 2] = o[dt][r4 * 4 + 2] * a0 + v.z * a1;
        o[dt][r4 * 4 + 3] = o[dt][r4 * 4 + 3] * a0 + v.w * a1;
      }
  }
  }

  // ---- epilogue: O = O^T / l, column col -> (row q0 + rq, head hq) ----
  // The wave's 32 x 128 bf16 tile goes through LDS (16-byte slots, slot of
  // (column, dims chunk c) = column * 16 + (c ^ (column & 15))) so that each
  // store instruction writes four whole 256-byte output rows.  The stores
  // carry the non-temporal hint: the output streams to memory while other
  // workgroups compute, instead of staying dirty in L2 for the write-back
  // at the kernel's end (measured: the Qwen2-7B batch 21.2 -> 20.0 us, the
  // same batch over an FP8 cache 24.8 -> 23.1 us).
  const float lt = l + __shfl_xor(l, 32);
  const float inv = bad ? __builtin_nanf("") : a.out_scale / lt;
  uint8_t* ot;                                    // this wave's 8 KiB in the (free) ring
  if constexpr (KG == 2) {
    ot = mg + 16 * 64 * 16 + 512;                 // after the merge data of the wave's stage
  } else {
    uint8_t* sg = (wave >> 1) == 0 ? st0 : (wave >> 1) == 1 ? st1 : (wave >> 1) == 2 ? st2 : st3;
    ot = sg + (wave & 1) * 8192;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c = dt * 4 + r4;                  // dims chunk of d = 8c + 4 hl .. + 3
      uint2 w;
      w.x = pack_bf16x2(o[dt][r4 * 4 + 0] * inv, o[dt][r4 * 4 + 1] * inv);
      w.y = pack_bf16x2(o[dt][r4 * 4 + 2] * inv, o[dt][r4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(ot + (col * 16 + (c ^ (col & 15))) * 16 + hl * 8) = w;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int idx = k * 64 + lane;
    const int oc = idx >> 4, c = idx & 15;        // column, dims chunk
    const uint4 v = *reinterpret_cast<const uint4*>(ot + (oc * 16 + (c ^ (oc & 15))) * 16);
    const int orow = q0 + oc % kBQ, oslot = HPW * hw + oc / kBQ;
    if (orow < n && oslot < G) {
      uint16_t* op = a.out + static_cast<int64_t>(r0 + orow) * a.out_stride +
                     static_cast<int64_t>(g * G + oslot) * kD + c * 8;
      const u32x4_t vv = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_t*>(op));
    }
  }
}

template <int KG, int WPG, int BS>
void launch_kg_bs(const PrefillKArgs& k, bool f8, size_t ids_bytes, hipStream_t stream) {
  const int64_t np = static_cast<int64_t>(k.num_kv_heads) * k.num_seqs;
  const int64_t slots = k.pairs_per_xcd > 0 ? int64_t{8} * k.pairs_per_xcd : np;
  const dim3 grid(static_cast<unsigned>(slots * k.num_qtiles));
  if (f8)
    hipLaunchKernelGGL((prefill_mfma_kernel<KG, WPG, true, BS>), grid, dim3(KG * WPG * 64),
                       ids_bytes, stream, k);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<KG, WPG, false, BS>), grid, dim3(KG * WPG * 64),
                       ids_bytes, stream, k);
}

// bs: log2 of the cache block size in 16-token blocks
template <int KG, int WPG>
void launch_kg(const PrefillKArgs& k, bool f8, int bs, size_t ids_bytes, hipStream_t stream) {
  switch (bs) {
    case 0: launch_kg_bs<KG, WPG, 0>(k, f8, ids_bytes, stream); break;
    case 1: launch_kg_bs<KG, WPG, 1>(k, f8, ids_bytes, stream); break;
    default: launch_kg_bs<KG, WPG, 2>(k, f8, ids_bytes, stream); break;
  }
}

}  // namespace

// One or two key groups.  Estimated time of each layout = max(longest work
// item, average work per CU) from measured costs on this GPU: a workgroup's
// start and finish (ids, first K/V tile, merge, stores) ~4 us with one group
// and ~5 us with two; a 32-key tile ~1.0 us (one group, 32 rows x G heads);
// a 64-key step ~1.5 us (two groups, 16 rows x 2 ceil(G/2) heads).  Only
// host-side maxima are known, so a row's keys are estimated from the longest
// context and chunk: c - n / 2 on average, c at most.  Two query heads per
// KV head always take one group: the two-group workgroup would have two
// waves issuing 16 loads each per step, and its 132 KB of stages leave one
// workgroup per CU where the one-group layout fits two (measured one-group
// wins: 55 against 64 us on a 512-row chunk at 1600 keys, 133 against 150 on
// a 64-row chunk at 4000).
int key_groups(const AttnArgs& a) {
  if (a.num_heads == 2 * a.num_kv_heads) return 1;
  const double c = a.max_context_len, n = a.max_query_len;
  const double rows = static_cast<double>(a.num_kv_heads) * a.num_tokens;   // (row, KV head) pairs
  const double avg_keys = c - 0.5 * n;
  const double cu = 256.0;
  const double t1 = std::max(4.0 + c / 32.0, rows / 32.0 * (4.0 + avg_keys / 32.0) / cu);
  const double t2 = std::max(5.0 + 1.5 * c / 64.0, rows / 16.0 * (5.0 + 1.5 * avg_keys / 64.0) / cu);
  return t2 < t1 ? 2 : 1;
}

// LDS a workgroup of the layout holds besides the block ids (the four
// stages, the scratch line and the flag; an upper bound)
static int lds_static_bytes(int kg) { return 4 * kg * kTile + 2048; }
// block ids a workgroup stages for contexts up to max_context_len
static int staged_ids(int kg, int max_context_len) {
  return 2 * kg * ((max_context_len + kg * kBK - 1) / (kg * kBK));
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  int KG = key_groups(a);
  // the block ids go to LDS beside the stages: past ~120K-token contexts
  // the two-group layout has no room for them and the one-group layout
  // (half the stage bytes) takes the call
  if (KG == 2 && staged_ids(2, a.max_context_len) * 4 > kLdsBytes - lds_static_bytes(2)) KG = 1;
  const int ids = staged_ids(KG, a.max_context_len);
  const bool mfma = a.dtype == kBF16 && a.head_dim == kD &&
                    (a.block_size == kB || a.block_size == 2 * kB || a.block_size == 4 * kB) &&
                    G >= 1 && G <= 8 && ids * 4 <= kLdsBytes - lds_static_bytes(KG);
  if (!mfma) return launch_attn_generic(a, stream);
  PrefillKArgs k{};
  k.q = static_cast<const uint16_t*>(a.q);
  k.q_stride = a.q_stride;
  k.k_cache = static_cast<const uint16_t*>(a.k_cache);
  k.v_cache = static_cast<const uint16_t*>(a.v_cache);
  k.num_blocks = a.num_blocks;
  k.cu_seqlens = a.cu_seqlens;
  k.context_lens = a.context_lens;
  k.block_tables = a.block_tables;
  k.max_blocks = a.max_blocks;
  k.out = static_cast<uint16_t*>(a.out);
  k.out_stride = a.out_stride;
  k.num_tokens = a.num_tokens;
  k.max_context_len = a.max_context_len;
  k.num_heads = a.num_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.num_seqs = a.num_seqs;
  const int rows = KG == 1 ? 32 : 16;
  k.num_qtiles = (a.max_query_len + rows - 1) / rows;
  const int np = a.num_kv_heads * a.num_seqs;
  // Pin each (KV head, sequence) pair to one XCD (its K/V stay in one L2)
  // with 32-row tiles, and with 16-row tiles only while an XCD holds one
  // pair: a long chunk then has up to twice as many tiles per pair, and
  // pinned beside another pair they outnumber the XCD's 32 CUs and run in
  // two rounds (a 512-row chunk beside two short ones: 53.7 us pinned, 31.9
  // spread).  The plain order spreads a pair's tiles over all XCDs.
  k.pairs_per_xcd = np >= 8 && (KG == 1 || np == 8) ? (np + 7) / 8 : 0;
  k.scale_log2 = a.scale * kLog2e * (a.cache_fp8 ? a.k_scale : 1.0f);
  k.out_scale = a.cache_fp8 ? a.v_scale : 1.0f;
  k.err = a.err;
  const int bs = a.block_size == 4 * kB ? 2 : a.block_size == 2 * kB ? 1 : 0;
  const bool f8 = a.cache_fp8 != 0;
  const size_t ids_bytes = static_cast<size_t>(ids) * 4;
  if (KG == 1) {
    switch (G) {
      case 1: launch_kg<1, 1>(k, f8, bs, ids_bytes, stream); break;
      case 2: launch_kg<1, 2>(k, f8, bs, ids_bytes, stream); break;
      case 3: launch_kg<1, 3>(k, f8, bs, ids_bytes, stream); break;
      case 4: launch_kg<1, 4>(k, f8, bs, ids_bytes, stream); break;
      case 5: launch_kg<1, 5>(k, f8, bs, ids_bytes, stream); break;
      case 6: launch_kg<1, 6>(k, f8, bs, ids_bytes, stream); break;
      case 7: launch_kg<1, 7>(k, f8, bs, ids_bytes, stream); break;
      default: launch_kg<1, 8>(k, f8, bs, ids_bytes, stream); break;
    }
  } else {
    switch ((G + 1) / 2) {
      case 1: launch_kg<2, 1>(k, f8, bs, ids_bytes, stream); break;
      case 2: launch_kg<2, 2>(k, f8, bs, ids_bytes, stream); break;
      case 3: launch_kg<2, 3>(k, f8, bs, ids_bytes, stream); break;
      default: launch_kg<2, 4>(k, f8, bs, ids_bytes, stream); break;
    }
  }
  return hipGetLastError();
}

}  // namespace qw
