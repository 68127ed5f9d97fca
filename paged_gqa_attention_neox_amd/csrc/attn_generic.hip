// Generic causal GQA attention over the paged cache, one query row and head
// per thread, fp32 arithmetic with an online (running-max) softmax.
//
// It serves the fp32 storage path, head_dim 64, and group sizes the tuned
// bf16 kernels do not instantiate; it is the plain, per-row statement of the
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
template <typename T> __device__ __forceinline__ T st(float v);
template <> __device__ __forceinline__ float st<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t st<uint16_t>(float v) { return f32_to_bf16(v); }

template <typename T, int D>
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
  if (row >= n) return;
  int c = a.context_lens[s];
  bool bad = c < 1 || c > a.max_context_len;   // contract: 1 <= c <= max_context_len
  if (bad) c = 0;
  const int pos = c - n + row;
  const int Hkv = a.num_kv_heads, B = a.block_size;
  const int g = h / (a.num_heads / Hkv);
  const int64_t t = static_cast<int64_t>(r0) + row;
  if (r0 < 0 || t >= a.num_tokens) return;       // rows outside the packed batch (bad cu_seqlens)
  const T* qp = static_cast<const T*>(a.q) + t * a.q_stride + static_cast<int64_t>(h) * D;
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = ld<T>(qp + e) * a.scale;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  bad = bad || pos < 0;
  for (int j = 0; j <= pos; ++j) {
    const int blk = bt[j / B];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      bad = true;
      break;
    }
    const int off = j % B;
    const T* kr = kc + ((static_cast<int64_t>(blk) * Hkv + g) * B + off) * D;
    float z = 0.0f;
#pragma unroll
    for (int e = 0; e < D; ++e) z = fmaf(qv[e], ld<T>(kr + e), z);
    const float mn = fmaxf(m, z);
    const float alpha = expf(m - mn);
    const float pz = expf(z - mn);
    l = fmaf(l, alpha, pz);
    const T* vr = vc + (static_cast<int64_t>(blk) * Hkv + g) * D * B + off;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = fmaf(acc[e], alpha, pz * ld<T>(vr + static_cast<int64_t>(e) * B));
    m = mn;
  }
  T* op = static_cast<T*>(a.out) + t * a.out_stride + static_cast<int64_t>(h) * D;
  const float inv = bad ? __builtin_nanf("") : 1.0f / l;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = st<T>(acc[e] * inv);
}

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream) {
  const int rows = a.cu_seqlens ? a.max_query_len : 1;
  const dim3 grid((rows + 63) / 64, a.num_heads, a.num_seqs);
  if (a.dtype == kBF16) {
    if (a.head_dim == 128) hipLaunchKernelGGL((attn_generic_kernel<uint16_t, 128>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((attn_generic_kernel<uint16_t, 64>), grid, dim3(64), 0, stream, a);
  } else {
    if (a.head_dim == 128) hipLaunchKernelGGL((attn_generic_kernel<float, 128>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((attn_generic_kernel<float, 64>), grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace qw
