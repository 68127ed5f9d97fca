// Generic causal GQA attention over the paged cache, one query row and head
// per thread, fp32 arithmetic with an online (running-max) softmax.
//
// It serves the fp32 storage path, head_dim 64, group sizes the tuned bf16
// kernels do not instantiate, and FP8 (E4M3FN) caches in prefill; it is the plain, per-row statement of the
// method: row i of a sequence with n new rows and context c sits at position
// c - n + i and attends to keys 0..c-n+i ("Qwen2大模型架构解析与vLLM优化实践",
// §7.3 causal mask; "Qwen 开源工程笔记", §3 varlen rows), head h reads KV
// head h / G ("Qwen2 模型结构代码详解", §2), keys are gathered through the
// block table ("vLLM 部署 Qwen", §2.1).
#include "common.h"
#include "kernels.h"

namespace qw {

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
// cache element: the storage type itself, or an E4M3FN code (uint8)
template <typename C> __device__ __forceinline__ float ldc(const C* p) { return ld<C>(p); }
template <> __device__ __forceinline__ float ldc<uint8_t>(const uint8_t* p) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<uint32_t>(*p), 0);
}
template <typename T> __device__ __forceinline__ T st(float v);
template <> __device__ __forceinline__ float st<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t st<uint16_t>(float v) { return f32_to_bf16(v); }

// C: cache element type (T, or uint8_t E4M3FN codes whose values are scaled
// by k_scale / v_scale: folded into the query scaling and the final divide)
template <typename T, typename C, int D>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int s = blockIdx.z, h = blockIdx.y;
  const int row = blockIdx.x * 64 + threadIdx.x;
  int r0, n;
  if (a.cu_seqlens) {
    r0 = a.cu_seqlens[s];
    n = a.cu_seqlens[s + 1] - r0;
  } else {
    r0 = s;
    n = 1;
  }
  // a row range outside the packed batch (bad cu_seqlens), a negative row
  // count or more rows than any valid context holds: flag, write no row
  if (r0 < 0 || n < 0 || static_cast<int64_t>(r0) + n > a.num_tokens || n > a.max_context_len) {
    if (row == 0) report_error(a.err, kErrSequence);
    return;
  }
  if (row >= n) return;
  int c = a.context_lens[s];
  bool bad = c < 1 || c > a.max_context_len;   // contract: 1 <= c <= max_context_len
  if (bad) report_error(a.err, kErrSequence);
  if (bad) c = 0;
  const int pos = c - n + row;
  const int Hkv = a.num_kv_heads, B = a.block_size;
  const int g = h / (a.num_heads / Hkv);
  const int64_t t = static_cast<int64_t>(r0) + row;
  const T* qp = static_cast<const T*>(a.q) + t * a.q_stride + static_cast<int64_t>(h) * D;
  const C* kc = static_cast<const C*>(a.k_cache);
  const C* vc = static_cast<const C*>(a.v_cache);
  const bool f8 = sizeof(C) == 1;
  const float qs = a.scale * (f8 ? a.k_scale : 1.0f);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = ld<T>(qp + e) * qs;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  if (pos < 0) report_error(a.err, kErrSequence);   // more rows than keys
  bad = bad || pos < 0;
  for (int j = 0; j <= pos; ++j) {
    const int blk = bt[j / B];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      bad = true;
      report_error(a.err, kErrBlock);
      break;
    }
    const int off = j % B;
    const C* kr = kc + ((static_cast<int64_t>(blk) * Hkv + g) * B + off) * D;
    float z = 0.0f;
#pragma unroll
    for (int e = 0; e < D; ++e) z = fmaf(qv[e], ldc<C>(kr + e), z);
    const float mn = fmaxf(m, z);
    const float alpha = expf(m - mn);
    const float pz = expf(z - mn);
    l = fmaf(l, alpha, pz);
    const C* vr = vc + (static_cast<int64_t>(blk) * Hkv + g) * D * B + off;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = fmaf(acc[e], alpha, pz * ldc<C>(vr + static_cast<int64_t>(e) * B));
    m = mn;
  }
  T* op = static_cast<T*>(a.out) + t * a.out_stride + static_cast<int64_t>(h) * D;
  const float inv = bad ? __builtin_nanf("") : (f8 ? a.v_scale : 1.0f) / l;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = st<T>(acc[e] * inv);
}

// The decode rows (one query row per sequence, no cu_seqlens): one
// workgroup per (sequence, query head).  Its four waves take the keys round
// robin; a wave's lanes hold D / 64 consecutive dims each, so a key's K row
// is one coalesced load per lane and its score the wave's sum of q_e k_e.
// Each wave keeps an online softmax state (m, l, acc); the four states are
// merged through LDS at the end (o = sum_w acc_w e^(m_w - M) / sum_w l_w
// e^(m_w - M)).  The per-thread kernel above walked a whole context in one
// thread per head.
template <typename T, typename C, int D>
__global__ __launch_bounds__(256) void attn_generic_decode_kernel(AttnArgs a) {
  constexpr int E = D / 64;                       // dims per lane
  constexpr int NW = 4;
  const int s = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ float sm[NW], sl[NW], sacc[NW][D];
  __shared__ int sbad;
  if (threadIdx.x == 0) sbad = 0;
  int c = a.context_lens[s];
  bool bad = c < 1 || c > a.max_context_len;     // contract: 1 <= c <= max_context_len
  if (bad && threadIdx.x == 0) report_error(a.err, kErrSequence);
  if (bad) c = 0;
  const int Hkv = a.num_kv_heads, B = a.block_size;
  const int g = h / (a.num_heads / Hkv);
  const bool f8 = sizeof(C) == 1;
  const float qs = a.scale * (f8 ? a.k_scale : 1.0f);
  const T* qp = static_cast<const T*>(a.q) + static_cast<int64_t>(s) * a.q_stride +
                static_cast<int64_t>(h) * D + lane * E;
  const C* kc = static_cast<const C*>(a.k_cache);
  const C* vc = static_cast<const C*>(a.v_cache);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  float qv[E], acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    qv[i] = ld<T>(qp + i) * qs;
    acc[i] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  bool wbad = false;
  __syncthreads();                                // sbad is set
  for (int j = w; j < c; j += NW) {               // wave-uniform
    const int blk = bt[j / B];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      wbad = true;
      break;
    }
    const int off = j % B;
    const C* kr = kc + ((static_cast<int64_t>(blk) * Hkv + g) * B + off) * D + lane * E;
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) z = fmaf(qv[i], ldc<C>(kr + i), z);
    z = wave_sum(z);
    const float mn = fmaxf(m, z);
    const float alpha = expf(m - mn);             // 0 for the first key (m = -inf)
    const float pz = expf(z - mn);
    l = fmaf(l, alpha, pz);
    const C* vr = vc + ((static_cast<int64_t>(blk) * Hkv + g) * D + lane * E) * B + off;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = fmaf(acc[i], alpha, pz * ldc<C>(vr + static_cast<int64_t>(i) * B));
    m = mn;
  }
  if (wbad && lane == 0) {
    report_error(a.err, kErrBlock);
    sbad = 1;
  }
  if (lane == 0) {
    sm[w] = m;
    sl[w] = l;
  }
#pragma unroll
  for (int i = 0; i < E; ++i) sacc[w][lane * E + i] = acc[i];
  __syncthreads();
  if (w != 0) return;
  float M = sm[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) M = fmaxf(M, sm[k]);
  float L = 0.0f, o[E];
#pragma unroll
  for (int i = 0; i < E; ++i) o[i] = 0.0f;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (sm[k] == -INFINITY) continue;             // a wave without keys
    const float wt = expf(sm[k] - M);
    L = fmaf(sl[k], wt, L);
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = fmaf(sacc[k][lane * E + i], wt, o[i]);
  }
  const float inv = bad || sbad ? __builtin_nanf("") : (f8 ? a.v_scale : 1.0f) / L;
  T* op = static_cast<T*>(a.out) + static_cast<int64_t>(s) * a.out_stride +
          static_cast<int64_t>(h) * D + lane * E;
#pragma unroll
  for (int i = 0; i < E; ++i) op[i] = st<T>(o[i] * inv);
}

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream) {
  const int rows = a.cu_seqlens ? a.max_query_len : 1;
  const dim3 grid((rows + 63) / 64, a.num_heads, a.num_seqs);
  const dim3 dgrid(a.num_seqs, a.num_heads);
#define QW_GEN(T, C, D)                                                                      \
  do {                                                                                       \
    if (a.cu_seqlens)                                                                        \
      hipLaunchKernelGGL((attn_generic_kernel<T, C, D>), grid, dim3(64), 0, stream, a);      \
    else                                                                                     \
      hipLaunchKernelGGL((attn_generic_decode_kernel<T, C, D>), dgrid, dim3(256), 0, stream, \
                         a);                                                                 \
  } while (0)
  const bool d128 = a.head_dim == 128;
  if (a.dtype == kBF16) {
    if (a.cache_fp8) { if (d128) QW_GEN(uint16_t, uint8_t, 128); else QW_GEN(uint16_t, uint8_t, 64); }
    else { if (d128) QW_GEN(uint16_t, uint16_t, 128); else QW_GEN(uint16_t, uint16_t, 64); }
  } else {
    if (a.cache_fp8) { if (d128) QW_GEN(float, uint8_t, 128); else QW_GEN(float, uint8_t, 64); }
    else { if (d128) QW_GEN(float, float, 128); else QW_GEN(float, float, 64); }
  }
#undef QW_GEN
  return hipGetLastError();
}

}  // namespace qw
