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
//   * key tiles of 32 keys (two cache blocks), double-buffered in LDS;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//     B = the wave's Q^T held in registers), so each lane owns one query
//     column: the softmax max and sum over keys are in-lane plus one
//     exchange between the two lane halves;
//   * online softmax in base 2 (scores pre-scaled by scale * log2 e), the
//     running output rescaled only when a column's max grows;
//   * O^T += V^T P^T with the same MFMA: P^T comes straight from the S^T
//     accumulator registers (rounded to bf16), V^T is read from LDS.  The K
//     rows feeding the MFMA are permuted (bits 2 and 3 of the key index
//     swapped) so that the keys each lane holds in P^T are 8 consecutive
//     keys, which the dims-major V cache tile stores contiguously;
//   * key tiles past the causal limit of the query tile are skipped, and the
//     grid is issued longest tile first.
// Other shapes and fp32 use the generic kernel.
#include "common.h"
#include "kernels.h"

namespace qw {

namespace {

constexpr int kD = 128;
constexpr int kB = 16;             // tokens per cache block
constexpr int kBQ = 32;            // query rows per tile
constexpr int kBK = 32;            // keys per tile
constexpr int kKRow = kD + 8;      // K tile row stride in LDS (elements): 272 B, conflict-free b128 reads
constexpr int kVRow = kBK + 8;     // V^T tile row stride in LDS (elements): 80 B
constexpr int kKTile = kBK * kKRow;    // elements
constexpr int kVTile = kD * kVRow;     // elements
constexpr int kChunks = 1024;          // 16-byte chunks per K+V tile (512 K + 512 V)
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PrefillKArgs {
  const uint16_t* q; int64_t q_stride;
  const uint16_t* k_cache; const uint16_t* v_cache; int num_blocks;
  const int32_t* cu_seqlens; const int32_t* context_lens;
  const int32_t* block_tables; int max_blocks;
  uint16_t* out; int64_t out_stride;
  int num_tokens, max_context_len, num_heads, num_kv_heads;
  float scale_log2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// key held by accumulator register r of a lane in half h (see the K row
// permutation above): 8 consecutive keys per 16-key chunk
__device__ __forceinline__ int key_of(int r, int h) { return (r & 7) + 8 * h + 16 * (r >> 3); }

template <int NW>
struct TileLoader {
  static constexpr int kPer = (kChunks + NW * 64 - 1) / (NW * 64);
  uint4 buf[kPer];

  // global -> registers for key tile kt
  __device__ __forceinline__ void load(const PrefillKArgs& a, const int32_t* bt, int nblk, int g,
                                       int kt, int tid, int ctx, bool& bad) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * NW * 64;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (i < kChunks) {
        const int kind = i >> 9;           // 0: K, 1: V
        const int w = i & 511;
        const int c = w >> 8;              // block within the tile
        const int lb = kt * 2 + c;         // logical block
        if (lb < nblk) {
          int blk = bt[lb];
          if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
            bad = true;
            blk = 0;
          }
          const int64_t tile = (static_cast<int64_t>(blk) * a.num_kv_heads + g) * (kB * kD);
          if (kind == 0) {
            const int row = (w & 255) >> 4, ch = w & 15;
            v = *reinterpret_cast<const uint4*>(a.k_cache + tile + row * kD + ch * 8);
          } else {
            const int d = (w & 255) >> 1, half = w & 1;
            v = *reinterpret_cast<const uint4*>(a.v_cache + tile + d * kB + half * 8);
            // V of keys past the context may hold anything (NaN): zero them,
            // a zero probability times NaN would poison every row
            const int key0 = kt * kBK + c * kB + half * 8;
            if (key0 + 8 > ctx) {
              uint32_t* e = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int k0 = key0 + 2 * q;
                uint32_t x = e[q];
                if (k0 >= ctx) x &= 0xffff0000u;
                if (k0 + 1 >= ctx) x &= 0x0000ffffu;
                e[q] = x;
              }
            }
          }
        }
      }
      buf[j] = v;
    }
  }

  __device__ __forceinline__ void store(uint16_t* kl, uint16_t* vl, int tid) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * NW * 64;
      if (i < kChunks) {
        const int w = i & 511;
        const int c = w >> 8;
        if ((i >> 9) == 0) {
          const int row = (w & 255) >> 4, ch = w & 15;
          *reinterpret_cast<uint4*>(kl + (c * kB + row) * kKRow + ch * 8) = buf[j];
        } else {
          const int d = (w & 255) >> 1, half = w & 1;
          *reinterpret_cast<uint4*>(vl + d * kVRow + c * kB + half * 8) = buf[j];
        }
      }
    }
  }
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void prefill_mfma_kernel(PrefillKArgs a) {
  const int g = blockIdx.x, s = blockIdx.y;
  const int qt = gridDim.z - 1 - blockIdx.z;    // longest (last) tiles first
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

  __shared__ __attribute__((aligned(16))) uint16_t sk[2][kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][kVTile];
  __shared__ int sbad;
  if (tid == 0) sbad = 0;

  // Q^T operand: column = query row q0 + col (clamped), 8 dims per k-step
  bf16x8_t qb[kD / 16];
  {
    const int row = min(q0 + col, n - 1);
    const uint16_t* qp = a.q + static_cast<int64_t>(r0 + row) * a.q_stride +
                         static_cast<int64_t>(hq) * kD + hl * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 16));
  }

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const int qpos = pos0 + q0 + col;

  // K row read by this lane for the S^T MFMA: MFMA row i = col holds key
  // perm(i) (bits 2 and 3 swapped)
  const int krow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);

  TileLoader<NW> ld;
  bool lbad = false;
  ld.load(a, bt, nblk, g, 0, tid, ctx, lbad);
  ld.store(sk[0], sv[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) ld.load(a, bt, nblk, g, kt + 1, tid, ctx, lbad);

    // ---- S^T = K Q^T ----
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint16_t* kp = &sk[cur][krow * kKRow + hl * 8];
    bf16x8_t ka[kD / 16];                       // all K fragments first: one LDS latency per tile
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) ka[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kp + ks * 16));
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qb[ks], acc, 0, 0, 0);
    // V fragments for this tile, read while the score MFMAs run
    bf16x8_t va[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t* vp = &sv[cur][(dt * 32 + col) * kVRow + hl * 8];
#pragma unroll
      for (int c = 0; c < 2; ++c) va[dt][c] = as_bf16x8(*reinterpret_cast<const uint4*>(vp + c * kB));
    }

    // ---- online softmax over this tile (base 2) ----
    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = acc[r] * a.scale_log2;
    if (kt * kBK + kBK - 1 > pos0 + q0) {        // diagonal tile: some key lies past some row
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = (kt * kBK + key_of(r, hl) <= qpos) ? sc[r] : -INFINITY;
    }
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    if (__builtin_amdgcn_ballot_w64(mnew > m) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m = mnew;
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[c * 8 + j] - m);
        l += p;
        pb[c][j] = static_cast<__bf16>(p);
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][c], pb[c], o[dt], 0, 0, 0);

    if (more) {
      // buffer cur^1 was last read in iteration kt-1, which every wave left
      // through the barrier below; one barrier per tile suffices
      ld.store(sk[cur ^ 1], sv[cur ^ 1], tid);
      __syncthreads();
    }
  }
  if (lbad) sbad = 1;
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
  const int tiles = (a.max_query_len + kBQ - 1) / kBQ;
  const dim3 grid(a.num_kv_heads, a.num_seqs, tiles);
  hipLaunchKernelGGL(prefill_mfma_kernel<NW>, grid, dim3(NW * 64), 0, stream, k);
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  const bool mfma = a.dtype == kBF16 && a.head_dim == kD && a.block_size == kB && G >= 1 && G <= 8;
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
