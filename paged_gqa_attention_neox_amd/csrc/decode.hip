// Paged single-token GQA decode for bf16, head_dim 128, block 16, with the
// context split into partitions ("split-K") and an exact log-sum-exp merge.
//
// Attention of one new token over its sequence's paged KV ("vLLM 部署 Qwen",
// §2.1 PagedAttention; §4.1: access to KV pages is what decode tuning is
// about).  GQA: the G = H/Hkv query heads of a group share one KV head
// ("Qwen2 模型结构代码详解", §2), so each (block, KV head) tile is read from HBM
// exactly once and used for all G heads.
//
// Work decomposition: one 256-thread workgroup (4 waves) per
// (partition of kPart tokens, KV head, sequence).  The waves take the
// partition's 16-token blocks round-robin.
//   Phase 1 (scores): K tile [16][128] bf16 = 4 KiB contiguous.  8 lanes per
//     key, 16 dims (32 B, two 128-bit loads) per lane; q.k with v_dot2 bf16
//     products accumulated in fp32, summed over the 8 lanes with DPP.  Scores
//     (pre-multiplied by scale * log2 e) go to LDS.
//   Phase 2 (softmax): per head max over the partition, p = 2^(z - max),
//     sum; p replaces the score in LDS.
//   Phase 3 (PV): V tile [128][16] bf16 (dims major).  Lane = 4 dims x 8
//     keys (four 128-bit loads); fp32 FMA with p broadcast from LDS.
//   Epilogue: combine key halves and waves; a single-partition sequence
//     writes its normalised output; otherwise the partial (max, sum, acc[d])
//     goes to the workspace and decode_reduce merges the partitions:
//       M = max_r m_r,  L = sum_r l_r 2^(m_r - M),  o = sum_r a_r 2^(m_r - M) / L
// The merge order depends only on logical positions, so results are
// bitwise reproducible and independent of the physical block placement.
#include "common.h"
#include "kernels.h"

namespace qw {

constexpr int kPart = 512;              // tokens per partition
constexpr int kBlk = 16;                // tokens per cache block
constexpr int kD = 128;                 // head_dim
constexpr int kPartBlocks = kPart / kBlk;
constexpr int kMaxG = 8;
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeKArgs {
  const uint16_t* q; int64_t q_stride;
  const uint16_t* k_cache; const uint16_t* v_cache; int num_blocks;
  const int32_t* block_tables; int max_blocks;
  const int32_t* context_lens;
  uint16_t* out; int64_t out_stride;
  float* ws_acc;   // [S][H][max_parts][128]
  float* ws_ml;    // [S][H][max_parts][2]  (max in log2 domain, sum)
  int num_heads, num_kv_heads, max_parts, max_context_len;
  float scale_log2;
};

// Context length of sequence s clamped to what the grid and workspace were
// sized for; *bad is set when the stored value breaks the contract.
__device__ __forceinline__ int checked_ctx(const DecodeKArgs& a, int s, bool* bad) {
  const int c = a.context_lens[s];
  *bad = c < 1 || c > a.max_context_len;
  return c < 1 ? 1 : (c > a.max_context_len ? a.max_context_len : c);
}

template <int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeKArgs a) {
  const int r = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  bool ctx_bad;
  const int ctx = checked_ctx(a, s, &ctx_bad);
  const int p0 = r * kPart;
  if (p0 >= ctx) return;
  const int ntok = min(kPart, ctx - p0);
  const int nblk = (ntok + kBlk - 1) / kBlk;
  const int nparts = (ctx + kPart - 1) / kPart;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int Hkv = a.num_kv_heads;

  __shared__ __attribute__((aligned(16))) float sc[kPart * 8];   // [token][8]
  __shared__ __attribute__((aligned(16))) float sacc[4][kMaxG * kD];
  __shared__ int sblk[kPartBlocks];
  __shared__ float sred[4][8];
  __shared__ float sM[8], sL[8];
  __shared__ int sbad;

  if (tid == 0) sbad = ctx_bad ? 1 : 0;
  __syncthreads();
  if (tid < nblk) {
    int b = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + (p0 / kBlk) + tid];
    if (static_cast<unsigned>(b) >= static_cast<unsigned>(a.num_blocks)) {
      sbad = 1;
      b = 0;
    }
    sblk[tid] = b;
  }
  __syncthreads();

  // ---------------- phase 1: scores ----------------
  {
    const int kr = lane >> 3;   // key within an 8-key round
    const int u = lane & 7;     // 16-dim slice
    uint4 qa[G], qb[G];
    const uint16_t* qp = a.q + static_cast<int64_t>(s) * a.q_stride +
                         static_cast<int64_t>(g * G) * kD + u * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qa[h] = *reinterpret_cast<const uint4*>(qp + h * kD);
      qb[h] = *reinterpret_cast<const uint4*>(qp + h * kD + 8);
    }
    for (int b = wave; b < nblk; b += 4) {
      const uint16_t* kb = a.k_cache + (static_cast<int64_t>(sblk[b]) * Hkv + g) * (kBlk * kD);
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int j = rd * 8 + kr;
        const uint4 k0 = *reinterpret_cast<const uint4*>(kb + j * kD + u * 16);
        const uint4 k1 = *reinterpret_cast<const uint4*>(kb + j * kD + u * 16 + 8);
        float acc[8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = dot2_bf16(qa[h].x, k0.x, 0.0f);
          x = dot2_bf16(qa[h].y, k0.y, x);
          x = dot2_bf16(qa[h].z, k0.z, x);
          x = dot2_bf16(qa[h].w, k0.w, x);
          x = dot2_bf16(qb[h].x, k1.x, x);
          x = dot2_bf16(qb[h].y, k1.y, x);
          x = dot2_bf16(qb[h].z, k1.z, x);
          x = dot2_bf16(qb[h].w, k1.w, x);
          acc[h] = sum8(x);
        }
        const int t = b * kBlk + j;
        if (u == 0) {
          const bool valid = t < ntok;
          float o[8];
#pragma unroll
          for (int h = 0; h < 8; ++h)
            o[h] = (h < G && valid) ? acc[h < G ? h : 0] * a.scale_log2 : -INFINITY;
          *reinterpret_cast<float4*>(&sc[t * 8]) = make_float4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<float4*>(&sc[t * 8 + 4]) = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: max, exp, sum over the partition ----------------
  {
    const int h = tid & 7;
    const int ch = tid >> 3;           // 32 token chunks
    const int tend = nblk * kBlk;
    float m = -INFINITY;
    for (int t = ch; t < tend; t += 32) m = fmaxf(m, sc[t * 8 + h]);
    m = fmaxf(m, __shfl_xor(m, 8));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane < 8) sred[wave][h] = m;
    __syncthreads();
    if (tid < 8) sM[tid] = fmaxf(fmaxf(sred[0][tid], sred[1][tid]), fmaxf(sred[2][tid], sred[3][tid]));
    __syncthreads();
    const float M = sM[h];
    float l = 0.0f;
    if (h < G) {
      for (int t = ch; t < tend; t += 32) {
        const float p = __builtin_amdgcn_exp2f(sc[t * 8 + h] - M);
        sc[t * 8 + h] = p;
        l += p;
      }
    }
    l += __shfl_xor(l, 8);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (lane < 8) sred[wave][h] = l;
    __syncthreads();
    if (tid < 8) sL[tid] = (sred[0][tid] + sred[1][tid]) + (sred[2][tid] + sred[3][tid]);
    __syncthreads();
  }

  // ---------------- phase 3: P V ----------------
  {
    const int e4 = (lane & 31) * 4;   // 4 dims
    const int kh = lane >> 5;         // key half (8 keys)
    float acc[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] = 0.0f;
    for (int b = wave; b < nblk; b += 4) {
      const uint16_t* vb = a.v_cache + (static_cast<int64_t>(sblk[b]) * Hkv + g) * (kBlk * kD);
      uint4 vr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[i] = *reinterpret_cast<const uint4*>(vb + (e4 + i) * kBlk + kh * 8);
      const bool full = (b + 1) * kBlk <= ntok;
      const int tb = b * kBlk + kh * 8;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float4 plo = *reinterpret_cast<const float4*>(&sc[(tb + kk) * 8]);
        const float4 phi = *reinterpret_cast<const float4*>(&sc[(tb + kk) * 8 + 4]);
        const float p[8] = {plo.x, plo.y, plo.z, plo.w, phi.x, phi.y, phi.z, phi.w};
        const bool live = full || (tb + kk < ntok);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = kk < 2 ? vr[i].x : kk < 4 ? vr[i].y : kk < 6 ? vr[i].z : vr[i].w;
          float v = (kk & 1) ? bf16_hi(w) : bf16_lo(w);
          v = live ? v : 0.0f;           // select: tail slots may hold NaN
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][i] = fmaf(p[h], v, acc[h][i]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] += __shfl_xor(acc[h][i], 32);
    if (kh == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        *reinterpret_cast<float4*>(&sacc[wave][h * kD + e4]) =
            make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    }
  }
  __syncthreads();

  // ---------------- epilogue ----------------
  const bool bad = sbad != 0;
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, e = idx % kD;
    float v = (sacc[0][idx] + sacc[1][idx]) + (sacc[2][idx] + sacc[3][idx]);
    if (bad) v = __builtin_nanf("");
    const int qh = g * G + h;
    if (nparts == 1) {
      a.out[static_cast<int64_t>(s) * a.out_stride + static_cast<int64_t>(qh) * kD + e] =
          f32_to_bf16(v / sL[h]);
    } else {
      a.ws_acc[((static_cast<int64_t>(s) * a.num_heads + qh) * a.max_parts + r) * kD + e] = v;
    }
  }
  if (nparts > 1 && tid < G) {
    const int qh = g * G + tid;
    float* ml = a.ws_ml + ((static_cast<int64_t>(s) * a.num_heads + qh) * a.max_parts + r) * 2;
    ml[0] = sM[tid];
    ml[1] = bad ? __builtin_nanf("") : sL[tid];
  }
}

// One 128-thread workgroup per (query head, sequence): merge the partitions.
__global__ __launch_bounds__(128) void decode_reduce_kernel(DecodeKArgs a) {
  const int qh = blockIdx.x, s = blockIdx.y, e = threadIdx.x;
  bool ctx_bad;
  const int ctx = checked_ctx(a, s, &ctx_bad);
  const int nparts = (ctx + kPart - 1) / kPart;
  if (nparts <= 1) return;
  const int64_t base = static_cast<int64_t>(s) * a.num_heads + qh;
  const float* ml = a.ws_ml + base * a.max_parts * 2;
  const float* acc = a.ws_acc + base * a.max_parts * kD;
  float M = -INFINITY;
  for (int r = 0; r < nparts; ++r) M = fmaxf(M, ml[2 * r]);
  float L = 0.0f, o = 0.0f;
  for (int r = 0; r < nparts; ++r) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * r] - M);
    L = fmaf(ml[2 * r + 1], w, L);
    o = fmaf(acc[static_cast<int64_t>(r) * kD + e], w, o);
  }
  a.out[static_cast<int64_t>(s) * a.out_stride + static_cast<int64_t>(qh) * kD + e] = f32_to_bf16(o / L);
}

DecodePlan plan_decode(int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, int dtype) {
  DecodePlan p{};
  const int G = num_heads / num_kv_heads;
  p.fast = dtype == kBF16 && head_dim == kD && block_size == kBlk && G >= 1 && G <= kMaxG;
  if (!p.fast) {
    p.ws_bytes = 0;
    return p;
  }
  p.part_tokens = kPart;
  p.max_parts = (max_context_len + kPart - 1) / kPart;
  if (p.max_parts <= 1) {
    p.ws_bytes = 0;
    return p;
  }
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * p.max_parts;
  p.ws_bytes = rows * kD * sizeof(float) + rows * 2 * sizeof(float);
  return p;
}

template <int G>
static void launch_partial(const DecodeKArgs& k, const AttnArgs& a, const DecodePlan& p,
                           hipStream_t stream) {
  const dim3 grid(p.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL(decode_partial_kernel<G>, grid, dim3(256), 0, stream, k);
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (!p.fast) return launch_attn_generic(a, stream);
  DecodeKArgs k{};
  k.q = static_cast<const uint16_t*>(a.q);
  k.q_stride = a.q_stride;
  k.k_cache = static_cast<const uint16_t*>(a.k_cache);
  k.v_cache = static_cast<const uint16_t*>(a.v_cache);
  k.num_blocks = a.num_blocks;
  k.block_tables = a.block_tables;
  k.max_blocks = a.max_blocks;
  k.context_lens = a.context_lens;
  k.out = static_cast<uint16_t*>(a.out);
  k.out_stride = a.out_stride;
  k.num_heads = a.num_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.max_parts = p.max_parts;
  k.max_context_len = a.max_context_len;
  k.scale_log2 = a.scale * kLog2e;
  if (p.max_parts > 1) {
    const size_t rows = static_cast<size_t>(a.num_seqs) * a.num_heads * p.max_parts;
    k.ws_acc = static_cast<float*>(a.workspace);
    k.ws_ml = k.ws_acc + rows * kD;
  }
  switch (a.num_heads / a.num_kv_heads) {
    case 1: launch_partial<1>(k, a, p, stream); break;
    case 2: launch_partial<2>(k, a, p, stream); break;
    case 3: launch_partial<3>(k, a, p, stream); break;
    case 4: launch_partial<4>(k, a, p, stream); break;
    case 5: launch_partial<5>(k, a, p, stream); break;
    case 6: launch_partial<6>(k, a, p, stream); break;
    case 7: launch_partial<7>(k, a, p, stream); break;
    default: launch_partial<8>(k, a, p, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_parts <= 1) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(a.num_heads, a.num_seqs), dim3(kD), 0, stream, k);
  return hipGetLastError();
}

}  // namespace qw
