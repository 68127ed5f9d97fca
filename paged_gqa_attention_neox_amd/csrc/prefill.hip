// Varlen causal GQA prefill over the paged cache on gfx950 matrix cores.
//
// What is computed: for each sequence s with n new rows and context c, row i
// (position c - n + i) of query head h attends to keys 0 .. c - n + i of KV
// head h / G ("Qwen2大模型架构解析与vLLM优化实践", §7.3 causal mask; "Qwen 开源
// 工程笔记", §3 packed varlen prefill; "Qwen2 模型结构代码详解", §2 GQA and
// scaling head_dim^-0.5), keys gathered through the block table ("vLLM 部署
// Qwen", §2.1).
//
// bf16, head_dim 128, block 16, group G <= 8:
//   * one workgroup per (KV head, 32-row query tile, sequence), one wave per
//     query head of the group: the K/V tiles of the group are staged in LDS
//     once and read by all G waves;
//   * key tiles of 32 keys (two cache blocks) stream through a ring of four
//     16 KB LDS stages with direct-to-LDS buffer loads (no register staging),
//     three tiles in flight; each wave issues the same number of 1 KB loads
//     per tile (surplus ones have an empty range and land in a scratch line),
//     so its outstanding-load count at every wait is a compile-time constant;
//   * the block ids the workgroup needs are staged in LDS once, so no load
//     inside the loop depends on another load;
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
// Other shapes and fp32 use the generic kernel.
#include "common.h"
#include "kernels.h"

namespace qw {

namespace {

constexpr int kD = 128;
constexpr int kB = 16;               // tokens per cache block
constexpr int kBQ = 32;              // query rows per tile
constexpr int kBK = 32;              // keys per tile
constexpr int kStage = 16384;        // bytes per LDS stage: K tile 8 KB + V^T tile 8 KB
constexpr int kLoads = 16;           // 1 KB direct-to-LDS loads per tile (8 K + 8 V)
constexpr int kBlockBytes = kB * kD * 2;   // one head's K (or V) of one cache block
constexpr int kMaxIds = 2048;        // block ids a workgroup stages (contexts up to 32K)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;        // raise the running max only past this margin (log2 units)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PrefillKArgs {
  const uint16_t* q; int64_t q_stride;
  const uint16_t* k_cache; const uint16_t* v_cache; int num_blocks;
  const int32_t* cu_seqlens; const int32_t* context_lens;
  const int32_t* block_tables; int max_blocks;
  uint16_t* out; int64_t out_stride;
  int num_tokens, max_context_len, num_heads, num_kv_heads;
  int num_seqs, num_qtiles, pairs_per_xcd;        // pairs_per_xcd 0: plain order
  float scale_log2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

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

// LDS layouts of one stage (16-byte slots):
//   K tile: slot(R, c) = R * 16 + (c ^ perm23(R & 15)), key R of the tile
//           (0..31), dims chunk c (8 dims, 0..15);
//   V^T tile (bytes 8192..): slot(b, d, h) = b * 256 + d * 2 + (h ^ vswz(d)),
//           cache block b of the tile, dims row d, 8-key half h.
// Load j (0..15) of a tile fills slots 64 j .. 64 j + 63: loads 0..7 the K
// tile (block j / 4), loads 8..15 the V^T tile (block (j - 8) / 4).  Byte
// offset inside the head's block tile of the chunk lane `lane` fetches:
__device__ __forceinline__ int load_offset(int j, int lane) {
  if (j < 8) {
    const int kk = 4 * (j & 3) + (lane >> 4);          // key within the cache block
    const int c = (lane & 15) ^ perm23(kk);
    return kk * (kD * 2) + c * 16;
  }
  const int u = ((j - 8) & 3) * 64 + lane;
  const int d = u >> 1;
  const int h = (u & 1) ^ vswz(d);
  return d * (kB * 2) + h * 16;
}

// 16 bytes per lane from buffer rs at byte offset voff into LDS at lds + 16 * lane
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void prefill_mfma_kernel(PrefillKArgs a) {
  constexpr int NI = (kLoads + NW - 1) / NW;      // loads per wave per tile
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
  const int g = p % a.num_kv_heads, s = p / a.num_kv_heads;
  const int qt = a.num_qtiles - 1 - z;            // longest (last) tiles first
  const int r0 = a.cu_seqlens[s];
  const int n = a.cu_seqlens[s + 1] - r0;
  const int q0 = qt * kBQ;
  if (q0 >= n) return;
  int ctx = a.context_lens[s];
  bool bad = ctx < n || ctx > a.max_context_len || r0 < 0 || r0 + n > a.num_tokens;
  if (bad) ctx = n;                               // keep every index in range; output is NaN
  if (r0 < 0 || r0 + n > a.num_tokens) return;    // rows not ours to write
  const int pos0 = ctx - n;                       // position of row 0
  const int qlast = min(q0 + kBQ, n) - 1;         // last valid row of the tile
  const int nkt = (pos0 + qlast) / kBK + 1;       // key tiles up to the causal limit
  const int nblk = (ctx + kB - 1) / kB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int hq = g * NW + wave;                   // query head of this wave
  const int hl = lane >> 5;                       // lane half
  const int col = lane & 31;                      // query column of this lane
  const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t trash[1024];
  __shared__ int sbad;
  __shared__ __attribute__((aligned(16))) int sids[kMaxIds];   // block ids of tiles 0 .. nkt-1

  // Q^T operand: column = query row q0 + col (clamped), 8 dims per k-step
  bf16x8_t qb[kD / 16];
  {
    const int row = min(q0 + col, n - 1);
    const uint16_t* qp = a.q + static_cast<int64_t>(r0 + row) * a.q_stride +
                         static_cast<int64_t>(hq) * kD + hl * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 16));
  }

  // stage the block ids; ids past the context or out of the pool read block 0
  {
    bool lbad = false;
    for (int i = tid; i < 2 * nkt; i += NW * 64) {
      int blk = 0;
      if (i < nblk) {
        blk = bt[i];
        if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
          lbad = true;
          blk = 0;
        }
      }
      sids[i] = blk;
    }
    if (tid == 0) sbad = 0;
    __syncthreads();
    if (lbad) sbad = 1;
  }

  // per-lane source offsets of this wave's loads (load j = wave + NW * i)
  int voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = wave + NW * i;
    voff[i] = j < kLoads ? load_offset(j, lane) : 0;
  }
  const int64_t head_off = static_cast<int64_t>(g) * (kB * kD);
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * (kB * kD);

  // issue the loads of key tile t into stage dst
  auto issue = [&](int t, uint8_t* dst) {
    const int2 ids = *reinterpret_cast<const int2*>(&sids[2 * t]);
    const int b0 = uniform(ids.x), b1 = uniform(ids.y);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = wave + NW * i;
      const bool live = j < kLoads;
      const int blk = ((j >> 2) & 1) ? b1 : b0;
      const uint16_t* base = ((j & 15) >= 8 ? a.v_cache : a.k_cache) + blk * blk_elems + head_off;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base), static_cast<short>(0), live ? kBlockBytes : 0, 0x00020000);
      uint8_t* l = live ? dst + j * 1024 : trash;
      load_lds16(rs, l, voff[i]);
    }
  };

  // V^T entries of keys >= ctx may hold anything (NaN): zero them, a zero
  // probability times NaN would poison the row
  auto sanitize = [&](int t, uint8_t* stg) {
    uint4* vt = reinterpret_cast<uint4*>(stg + 8192);
    for (int sl = tid; sl < 512; sl += NW * 64) {
      const int b = sl >> 8, u = sl & 255, d = u >> 1;
      const int h = (u & 1) ^ vswz(d);
      const int key0 = t * kBK + b * kB + h * 8;
      if (key0 + 8 > ctx) {
        uint4 v = vt[sl];
        uint32_t* e = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k0 = key0 + 2 * q;
          uint32_t x = e[q];
          if (k0 >= ctx) x &= 0xffff0000u;
          if (k0 + 1 >= ctx) x &= 0x0000ffffu;
          e[q] = x;
        }
        vt[sl] = v;
      }
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;                  // running max (log2 units), sum
  const int qpos = pos0 + q0 + col;
  const float c2 = a.scale_log2;

  // K row read by this lane for the S^T MFMA: MFMA row i = col holds key
  // perm23(i) of the tile; its dims chunk c sits in slot c ^ (col & 15)
  const int krow = (col & 16) | perm23(col & 15);
  const int kx = hl ^ (col & 15);
  const int vlane = (col * 2 + (hl ^ vswz(col))) * 16;
  const int sani_tile = (ctx % kBK) ? ctx / kBK : -1;   // tile holding keys >= ctx

  // S^T = K Q^T of the key tile in stage stg
  auto qk = [&](const uint8_t* stg) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint8_t* kp = stg + krow * (kD * 2);
    bf16x8_t ka[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      ka[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kp + ((2 * ks) ^ kx) * 16));
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qb[ks], acc, 0, 0, 0);
    return acc;
  };

  // causal mask of a diagonal tile (some key lies past some row of the tile)
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
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * c2;
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
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c * 8 + j], c2, -m));
        lt += p;
        pb[c][j] = static_cast<__bf16>(p);
      }
    }
    l = l * alpha + lt;
    return alpha;
  };

  // O^T = alpha O^T + V^T P^T for the key tile in stage stg
  auto pv = [&](float alpha, const uint8_t* stg) {
    bf16x8_t va[4][2];
    const uint8_t* vp = stg + 8192 + vlane;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        va[dt][c] = as_bf16x8(*reinterpret_cast<const uint4*>(vp + c * 4096 + dt * 1024));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][c], pb[c], o[dt], 0, 0, 0);
  };

  // one key tile: wait until it is in LDS for every wave (the waits leave
  // the loads of later tiles outstanding), refill the stage of tile kt - 1
  // (every wave passed the barrier, so it finished with it) with tile
  // kt + 3, then scores, softmax and PV of tile kt
  auto step = [&](int kt, uint8_t* cur, uint8_t* refill) {
    if (kt + 2 < nkt) wait_vm<2 * NI>();
    else if (kt + 1 < nkt) wait_vm<NI>();
    else wait_vm<0>();
    barrier();
    if (kt == sani_tile) {
      sanitize(kt, cur);
      wait_lds();
      barrier();
    }
    if (kt + 3 < nkt) issue(kt + 3, refill);
    f32x16_t sc = qk(cur);
    mask(kt, sc);
    const float alpha = softmax(sc);
    pv(alpha, cur);
  };

  issue(0, st0);
  if (nkt > 1) issue(1, st1);
  if (nkt > 2) issue(2, st2);
  for (int kt = 0; kt < nkt; kt += 4) {
    step(kt, st0, st3);
    if (kt + 1 >= nkt) break;
    step(kt + 1, st1, st0);
    if (kt + 2 >= nkt) break;
    step(kt + 2, st2, st1);
    if (kt + 3 >= nkt) break;
    step(kt + 3, st3, st2);
  }
  __syncthreads();
  if (sbad) bad = true;

  // ---- epilogue: O = O^T / l, column col -> row q0 + col ----
  const float lt = l + __shfl_xor(l, 32);
  const float inv = bad ? __builtin_nanf("") : 1.0f / lt;
  const int row = q0 + col;
  if (row < n) {
    uint16_t* op = a.out + static_cast<int64_t>(r0 + row) * a.out_stride + static_cast<int64_t>(hq) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = dt * 32 + r4 * 8 + hl * 4;
        uint2 w;
        w.x = pack_bf16x2(o[dt][r4 * 4 + 0] * inv, o[dt][r4 * 4 + 1] * inv);
        w.y = pack_bf16x2(o[dt][r4 * 4 + 2] * inv, o[dt][r4 * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + d) = w;
      }
    }
  }
}

template <int NW>
void launch_nw(const PrefillKArgs& k, const AttnArgs& a, hipStream_t stream) {
  const int64_t np = static_cast<int64_t>(a.num_kv_heads) * a.num_seqs;
  const int64_t slots = k.pairs_per_xcd > 0 ? int64_t{8} * k.pairs_per_xcd : np;
  const dim3 grid(static_cast<unsigned>(slots * k.num_qtiles));
  hipLaunchKernelGGL(prefill_mfma_kernel<NW>, grid, dim3(NW * 64), 0, stream, k);
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  const int ids = 2 * ((a.max_context_len + kBK - 1) / kBK);
  const bool mfma = a.dtype == kBF16 && a.head_dim == kD && a.block_size == kB && G >= 1 &&
                    G <= 8 && ids <= kMaxIds;
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
  k.num_qtiles = (a.max_query_len + kBQ - 1) / kBQ;
  const int np = a.num_kv_heads * a.num_seqs;
  k.pairs_per_xcd = np >= 8 ? (np + 7) / 8 : 0;
  k.scale_log2 = a.scale * kLog2e;
  switch (G) {
    case 1: launch_nw<1>(k, a, stream); break;
    case 2: launch_nw<2>(k, a, stream); break;
    case 3: launch_nw<3>(k, a, stream); break;
    case 4: launch_nw<4>(k, a, stream); break;
    case 5: launch_nw<5>(k, a, stream); break;
    case 6: launch_nw<6>(k, a, stream); break;
    case 7: launch_nw<7>(k, a, stream); break;
    default: launch_nw<8>(k, a, stream); break;
  }
  return hipGetLastError();
}

}  // namespace qw
