// Paged single-token GQA decode for bf16, head_dim 128, block 16, with the
// context split into partitions ("split-K") and an exact log-sum-exp merge.
// The cache may hold bf16 or FP8 E4M3FN codes ("Qwen2大模型架构解析与vLLM优化
// 实践", §4.1-4.2 FP8 KV-cache quantization with cache scales, §6.3 E4M3FN):
// FP8 tiles are half the bytes and are widened to bf16 pairs in registers
// (exact), k_scale folds into the score scale and v_scale into the output.
//
// Attention of one new token over its sequence's paged KV ("vLLM 部署 Qwen",
// §2.1 PagedAttention; §4.1: access to KV pages is what decode tuning is
// about).  GQA: the G = H/Hkv query heads of a group share one KV head
// ("Qwen2 模型结构代码详解", §2), so each (block, KV head) tile is read from HBM
// exactly once and used for all G heads.
//
// Work decomposition: one 256-thread workgroup (4 waves) per
// (partition of kPart tokens, KV head, sequence).  The waves take the
// partition's 16-token blocks round-robin and stream them through kNBuf
// register buffers, so the next blocks' loads are always in flight.
//   Phase 1 (scores): K tile [16][128] bf16 = 4 KiB contiguous.  8 lanes per
//     key, 16 dims (two 128-bit loads) per lane; q.k with v_dot2 bf16
//     products accumulated in fp32, summed over the 8 lanes with DPP.  Raw
//     scores go to LDS (the scale is applied in the softmax).
//   Phase 2 (softmax): per head max over the partition; p = 2^((z - max)
//     * scale * log2 e) rounded to bf16 and stored as pairs of consecutive tokens; the sum of
//     the rounded p.  The first V tile is already loading.
//   Phase 3 (PV): V tile [128][16] bf16 (dims major), so a 32-bit word holds
//     two consecutive tokens of one dim: acc += v_dot2(p pair, v pair), fp32
//     accumulation.  Lane = 4 dims x 8 tokens (four 128-bit loads).  Every
//     128-bit load instruction of a wave reads 1 KiB of a tile contiguously.
//   Epilogue: combine key halves and waves; a single-partition sequence
//     writes its normalised output; otherwise the partial (max, sum, acc[d])
//     goes to the workspace and decode_reduce merges the partitions:
//       M = max_r m_r,  L = sum_r l_r 2^(m_r - M),  o = sum_r a_r 2^(m_r - M) / L
// The merge order depends only on logical positions, so results are
// bitwise reproducible and independent of the physical block placement.
#include "common.h"
#include "kernels.h"

namespace qw {

#ifndef QW_DECODE_PART
#define QW_DECODE_PART 512
#endif
#ifndef QW_DECODE_NW
#define QW_DECODE_NW 4
#endif
constexpr int kPart = QW_DECODE_PART;   // tokens per partition
constexpr int kNW = QW_DECODE_NW;       // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kBlk = 16;                // tokens per cache block
constexpr int kD = 128;                 // head_dim
constexpr int kPartBlocks = kPart / kBlk;
constexpr int kMaxG = 8;
#ifndef QW_DECODE_NBUF
#define QW_DECODE_NBUF 2
#endif
constexpr int kNBuf = QW_DECODE_NBUF;   // blocks of K (or V) in flight per wave
constexpr float kLog2e = 1.4426950408889634f;

// gfx9-family buffer descriptor word 3 (raw 32-bit accesses, no swizzle)
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ uint4 ld_buf16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ uint2 ld_buf8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
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
  const int32_t* context_lens;
  uint16_t* out; int64_t out_stride;
  float* ws_acc;   // [S][H][max_parts][128]
  float* ws_ml;    // [S][H][max_parts][2]  (max in log2 domain, sum)
  int num_heads, num_kv_heads, max_parts, max_context_len;
  float scale_log2;   // scale * log2 e (* k_scale with an FP8 cache)
  float out_scale;    // 1, or v_scale with an FP8 cache
};

// Context length of sequence s clamped to what the grid and workspace were
// sized for; *bad is set when the stored value breaks the contract.
__device__ __forceinline__ int checked_ctx(const DecodeKArgs& a, int s, bool* bad) {
  const int c = a.context_lens[s];
  *bad = c < 1 || c > a.max_context_len;
  return c < 1 ? 1 : (c > a.max_context_len ? a.max_context_len : c);
}

#ifndef QW_DECODE_WAVES
#define QW_DECODE_WAVES 4
#endif

// F8: the caches hold E4M3FN codes (K tile 2 KiB, V tile 2 KiB); they are
// widened to bf16 pairs in registers and the same arithmetic follows.
template <int G, bool F8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(QW_DECODE_WAVES)))
void decode_partial_kernel(DecodeKArgs a) {
  constexpr int kEl = F8 ? 1 : 2;                 // bytes per cache element
  constexpr int kTileBytes = kBlk * kD * kEl;
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

  // scores [token][8 heads] (fp32); after the softmax the same space holds
  // the per-wave partial outputs of the merge
  __shared__ __attribute__((aligned(16))) float sc[kPart * 8];
  // probabilities as bf16 pairs of consecutive tokens: [token pair][8 heads]
  __shared__ __attribute__((aligned(16))) uint32_t sp2[kPart / 2 * 8];
  __shared__ int sblk[kPartBlocks];
  __shared__ float sred[kNW][8];
  __shared__ float sM[8], sL[8];
  __shared__ int sbad;
  float (*sacc)[kMaxG * kD] = reinterpret_cast<float (*)[kMaxG * kD]>(sc);
  static_assert(kNW * kMaxG * kD <= kPart * 8, "merge buffer must fit in the score buffer");

  if (tid == 0) sbad = ctx_bad ? 1 : 0;
  __syncthreads();
  for (int i = tid; i < nblk; i += kThreads) {
    int b = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + (p0 / kBlk) + i];
    if (static_cast<unsigned>(b) >= static_cast<unsigned>(a.num_blocks)) {
      sbad = 1;
      b = 0;
    }
    sblk[i] = b;
  }
  __syncthreads();

  // Blocks of this wave: b = wave + kNW i, i < nbw.
  const int nbw = nblk > wave ? (nblk - wave + kNW - 1) / kNW : 0;
  // Lane roles.  Each 128-bit load instruction of a wave reads 1 KiB of one
  // tile contiguously.
  //   phase 1: key kr of an 8-key round; dims 8u..8u+7 and 64+8u..64+8u+7
  //            (FP8: dims 16u..16u+15, one 16-byte load)
  //   phase 3: dims d0 + 32 i (i < 4); keys 8 kh .. 8 kh + 7 of the block
  const int kr = lane >> 3;
  const int u = lane & 7;
  const int d0 = lane >> 1;
  const int kh = lane & 1;
  // Tiles are read with buffer loads through a per-tile descriptor (uniform,
  // in SGPRs).  Every pipeline load is issued unconditionally so the number
  // of loads in flight is static and each wait covers exactly one block; a
  // prefetch past the wave's last block gets a zero-size descriptor, which
  // returns zeros without touching memory.
  auto rsrc = [&](const uint8_t* base, int i) {
    const bool live = i < nbw;
    const int b = uniform(sblk[wave + kNW * (live ? i : 0)]);
    const uint8_t* t = base + (static_cast<int64_t>(b) * Hkv + g) * kTileBytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(t), static_cast<short>(0),
                                             live ? kTileBytes : 0, kBufferFlags);
  };
  // byte offsets within a tile (bf16 K: key kr, dims 8u.. and 64+8u..; FP8 K:
  // key kr, dims 16u..16u+15; V: dims d0 + 32 i, keys 8 kh..8 kh+7)
  const int koff = F8 ? kr * kD + u * 16 : (kr * kD + u * 8) * 2;
  const int voff = F8 ? d0 * kBlk + kh * 8 : lane * 16;
  auto load_k = [&](int i, uint4 (&buf)[4]) {
    const auto r = rsrc(a.k_cache, i);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      if constexpr (F8) {
        buf[rd] = ld_buf16(r, koff + rd * 8 * kD);
      } else {
        buf[2 * rd] = ld_buf16(r, koff + rd * 8 * kD * 2);
        buf[2 * rd + 1] = ld_buf16(r, koff + rd * 8 * kD * 2 + 128);
      }
    }
  };
  auto load_v = [&](int i, uint4 (&buf)[4]) {
    const auto r = rsrc(a.v_cache, i);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (F8) {
        const uint2 c = ld_buf8(r, voff + d * 32 * kBlk);
        buf[d] = make_uint4(c.x, c.y, 0u, 0u);
      } else {
        buf[d] = ld_buf16(r, voff + d * 1024);
      }
    }
  };

  // ---------------- phase 1: raw scores q.k ----------------
  uint4 vbuf[kNBuf][4];
  {
    uint4 qa[G], qb[G];
    const uint16_t* qp = a.q + static_cast<int64_t>(s) * a.q_stride +
                         static_cast<int64_t>(g * G) * kD + (F8 ? u * 16 : u * 8);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qa[h] = *reinterpret_cast<const uint4*>(qp + h * kD);
      qb[h] = *reinterpret_cast<const uint4*>(qp + h * kD + (F8 ? 8 : 64));
    }
    auto scores = [&](int i, const uint4 (&kbuf)[4]) {
      const int b = wave + kNW * i;
      const bool full = (b + 1) * kBlk <= ntok;
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        uint4 k0, k1;
        if constexpr (F8) {
          k0 = fp8x8_to_bf16x8(make_uint2(kbuf[rd].x, kbuf[rd].y));
          k1 = fp8x8_to_bf16x8(make_uint2(kbuf[rd].z, kbuf[rd].w));
        } else {
          k0 = kbuf[2 * rd];
          k1 = kbuf[2 * rd + 1];
        }
        float acc[8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = dot2_bf16_first(qa[h].x, k0.x);
          x = dot2_bf16(qa[h].y, k0.y, x);
          x = dot2_bf16(qa[h].z, k0.z, x);
          x = dot2_bf16(qa[h].w, k0.w, x);
          x = dot2_bf16(qb[h].x, k1.x, x);
          x = dot2_bf16(qb[h].y, k1.y, x);
          x = dot2_bf16(qb[h].z, k1.z, x);
          x = dot2_bf16(qb[h].w, k1.w, x);
          acc[h] = sum8(x);
        }
#pragma unroll
        for (int h = G; h < 8; ++h) acc[h] = -INFINITY;
        const int t = b * kBlk + rd * 8 + kr;
        if (!full) {                      // the partition's last block: keys past the context
          if (t >= ntok) {                // (slots there may hold NaN) are excluded by select
#pragma unroll
            for (int h = 0; h < 8; ++h) acc[h] = -INFINITY;
          }
        }
        if (u == 0) {
          *reinterpret_cast<float4*>(&sc[t * 8]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
          *reinterpret_cast<float4*>(&sc[t * 8 + 4]) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
      }
    };
    uint4 kbuf[kNBuf][4];
#pragma unroll
    for (int j = 0; j < kNBuf - 1; ++j) load_k(j, kbuf[j]);
    for (int i = 0; i < nbw; i += kNBuf) {
#pragma unroll
      for (int j = 0; j < kNBuf; ++j) {
        load_k(i + j + kNBuf - 1, kbuf[(j + kNBuf - 1) % kNBuf]);
        if (i + j < nbw) scores(i + j, kbuf[j]);
      }
    }
    // the first V tiles of this wave: in flight across the softmax phase
#pragma unroll
    for (int j = 0; j < kNBuf - 1; ++j) load_v(j, vbuf[j]);
  }
  __syncthreads();

  // ---------------- phase 2: max, p (bf16 pairs), sum ----------------
  {
    const int h = tid & 7;
    const int ch = tid >> 3;           // kNW * 8 chunks
    constexpr int kCh = kNW * 8;
    const int tend = nblk * kBlk;
    float m = -INFINITY;
    for (int t = ch; t < tend; t += kCh) m = fmaxf(m, sc[t * 8 + h]);
    m = fmaxf(m, __shfl_xor(m, 8));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane < 8) sred[wave][h] = m;
    __syncthreads();
    if (tid < 8) {
      float mm = sred[0][tid];
#pragma unroll
      for (int w = 1; w < kNW; ++w) mm = fmaxf(mm, sred[w][tid]);
      sM[tid] = mm;
    }
    __syncthreads();
    // p = 2^((z - max) * scale * log2 e): the raw-score max is the scaled max
    const float c = a.scale_log2;
    const float mc = -sM[h] * c;
    float l = 0.0f;
    if (h < G) {
      // the normaliser sums the rounded weights that P V will use
      for (int j = ch; j < tend / 2; j += kCh) {
        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[(2 * j) * 8 + h], c, mc)),
                                       __builtin_amdgcn_exp2f(fmaf(sc[(2 * j + 1) * 8 + h], c, mc)));
        sp2[j * 8 + h] = w;
        l += bf16_lo(w) + bf16_hi(w);
      }
    }
    l += __shfl_xor(l, 8);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (lane < 8) sred[wave][h] = l;
    __syncthreads();
    if (tid < 8) {
      float ll = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) ll += sred[w][tid];
      sL[tid] = ll;
      sM[tid] *= c;                    // partition max in the log2 domain for the merge
    }
    // (sp2 is complete: the barrier above came after every write)
  }

  // ---------------- phase 3: P V with bf16 pairs ----------------
  {
    float acc[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] = 0.0f;
    auto pv = [&](int i, uint4 (&vr)[4]) {
      const int b = wave + kNW * i;
      if constexpr (F8) {
#pragma unroll
        for (int d = 0; d < 4; ++d) vr[d] = fp8x8_to_bf16x8(make_uint2(vr[d].x, vr[d].y));
      }
      const int pair0 = (b * kBlk + kh * 8) / 2;     // first token pair of this lane half
      if ((b + 1) * kBlk > ntok) {                   // last block: tail slots may hold NaN
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t* w = reinterpret_cast<uint32_t*>(&vr[d]);
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const int t0 = 2 * (pair0 + pp);
            w[pp] = t0 >= ntok ? 0u : (t0 + 1 >= ntok ? (w[pp] & 0xffffu) : w[pp]);
          }
        }
      }
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint4 plo = *reinterpret_cast<const uint4*>(&sp2[(pair0 + pp) * 8]);
        const uint4 phi = *reinterpret_cast<const uint4*>(&sp2[(pair0 + pp) * 8 + 4]);
        const uint32_t p[8] = {plo.x, plo.y, plo.z, plo.w, phi.x, phi.y, phi.z, phi.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t w = pp == 0 ? vr[d].x : pp == 1 ? vr[d].y : pp == 2 ? vr[d].z : vr[d].w;
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][d] = dot2_bf16(p[h], w, acc[h][d]);
        }
      }
    };
    for (int i = 0; i < nbw; i += kNBuf) {
#pragma unroll
      for (int j = 0; j < kNBuf; ++j) {
        load_v(i + j + kNBuf - 1, vbuf[(j + kNBuf - 1) % kNBuf]);
        if (i + j < nbw) pv(i + j, vbuf[j]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] += dpp<kDppXor1>(acc[h][i]);   // the other key half
    // sc (aliased by sacc) is no longer read by anyone: phase 2 ended with a barrier
    if (kh == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[wave][h * kD + d0 + 32 * i] = acc[h][i];
    }
  }
  __syncthreads();

  // ---------------- epilogue ----------------
  const bool bad = sbad != 0;
  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int h = idx / kD, e = idx % kD;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) v += sacc[w][idx];
    if (bad) v = __builtin_nanf("");
    const int qh = g * G + h;
    if (nparts == 1) {
      a.out[static_cast<int64_t>(s) * a.out_stride + static_cast<int64_t>(qh) * kD + e] =
          f32_to_bf16(v * a.out_scale / sL[h]);
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

// Merge of the partitions: one 128-thread workgroup per (query head,
// sequence), one output element per thread.  Partitions are taken 64 at a
// time: their (m, l) pairs go to LDS in one round of loads, the weights
// 2^(m_r - M) follow from the running maximum, and every thread issues the
// loads of its 64 partial sums back to back, so the merge pays a few memory
// latencies instead of one per partition.
constexpr int kMergeBatch = 64;

__global__ __launch_bounds__(128) void decode_reduce_kernel(DecodeKArgs a) {
  const int qh = blockIdx.x, s = blockIdx.y, e = threadIdx.x;
  bool ctx_bad;
  const int ctx = checked_ctx(a, s, &ctx_bad);
  const int nparts = (ctx + kPart - 1) / kPart;
  if (nparts <= 1) return;
  __shared__ float sm[kMergeBatch], sl[kMergeBatch];
  __shared__ float sred[2];
  const int64_t base = static_cast<int64_t>(s) * a.num_heads + qh;
  const float* ml = a.ws_ml + base * a.max_parts * 2;
  const float* acc = a.ws_acc + base * a.max_parts * kD + e;

  float M = -INFINITY, L = 0.0f, o = 0.0f;      // running over batches (uniform)
  for (int c0 = 0; c0 < nparts; c0 += kMergeBatch) {
    const int cn = min(kMergeBatch, nparts - c0);
    float x[kMergeBatch];
#pragma unroll
    for (int r = 0; r < kMergeBatch; ++r) x[r] = r < cn ? acc[static_cast<int64_t>(c0 + r) * kD] : 0.0f;
    if (e < cn) {
      sm[e] = ml[2 * (c0 + e)];
      sl[e] = ml[2 * (c0 + e) + 1];
    }
    __syncthreads();
    if (e < 64) {                                // wave 0: batch max
      float mb = e < cn ? sm[e] : -INFINITY;
      mb = wave_max(mb);
      if (e == 0) sred[0] = mb;
    }
    __syncthreads();
    const float Mn = fmaxf(M, sred[0]);
    const float alpha = M > -INFINITY ? __builtin_amdgcn_exp2f(M - Mn) : 0.0f;
    float lb = 0.0f, ob = 0.0f;
#pragma unroll
    for (int r = 0; r < kMergeBatch; ++r) {
      if (r < cn) {
        const float w = __builtin_amdgcn_exp2f(sm[r] - Mn);
        lb = fmaf(sl[r], w, lb);
        ob = fmaf(x[r], w, ob);
      }
    }
    L = fmaf(L, alpha, lb);
    o = fmaf(o, alpha, ob);
    M = Mn;
    __syncthreads();                             // sm/sl reused by the next batch
  }
  a.out[static_cast<int64_t>(s) * a.out_stride + static_cast<int64_t>(qh) * kD + e] =
      f32_to_bf16(ctx_bad ? __builtin_nanf("") : o * a.out_scale / L);
}

DecodePlan plan_decode(int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, int dtype, int cache_fp8) {
  (void)cache_fp8;                    // both cache formats have the split-K kernel
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
  if (a.cache_fp8)
    hipLaunchKernelGGL((decode_partial_kernel<G, true>), grid, dim3(kThreads), 0, stream, k);
  else
    hipLaunchKernelGGL((decode_partial_kernel<G, false>), grid, dim3(kThreads), 0, stream, k);
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (!p.fast) return launch_attn_generic(a, stream);
  DecodeKArgs k{};
  k.q = static_cast<const uint16_t*>(a.q);
  k.q_stride = a.q_stride;
  k.k_cache = static_cast<const uint8_t*>(a.k_cache);
  k.v_cache = static_cast<const uint8_t*>(a.v_cache);
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
  k.scale_log2 = a.scale * kLog2e * (a.cache_fp8 ? a.k_scale : 1.0f);
  k.out_scale = a.cache_fp8 ? a.v_scale : 1.0f;
  if (p.max_parts > 1) {
    const size_t rows = static_cast<size_t>(a.num_seqs) * a.num_heads * p.max_parts;
    k.ws_acc = static_cast<float*>(a.workspace);
    k.ws_ml = k.ws_acc + rows * kD;
  }
  const int G = a.num_heads / a.num_kv_heads;
  switch (G) {
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
