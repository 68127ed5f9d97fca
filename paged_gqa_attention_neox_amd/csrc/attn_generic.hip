// Generic causal GQA attention over the paged cache, fp32 arithmetic with an
// online (running-max) softmax, one wave per query row and head.
//
// It serves the fp32 storage path, head_dim 64, group sizes the tuned bf16
// kernels do not instantiate, and FP8 (E4M3FN) caches in prefill beyond the
// MFMA kernel's shapes.  Row i of a sequence with n new rows and context c
// sits at position c - n + i and attends to keys 0..c-n+i
// ("Qwen2大模型架构解析与vLLM优化实践", §7.3 causal mask; "Qwen 开源工程笔记", §3
// varlen rows), head h reads KV head h / G ("Qwen2 模型结构代码详解", §2), keys
// are gathered through the block table ("vLLM 部署 Qwen", §2.1).
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

constexpr int kChunk = 16;                        // keys per chunk (block sizes are multiples)

// One wave attends keys j0 .. j0 + 15 of (cache tile `tile`, 16-key run at
// offset off0 of its block); keys at or past kend are masked by selection
// (their slots may hold anything).  A lane holds dims lane E .. lane E + E - 1
// (E = D / 64) of q and of the output state (m, l, acc).  Every K and V load
// of the chunk is issued at once.  The 16 partial dots are summed over the
// wave by a butterfly: at each exchange over lane bits 5..2 a lane keeps the
// half of its keys that bit selects, summed with its partner's (8 + 4 + 2 +
// 1 shuffles); two more exchanges over bits 1 and 0 leave key k's score in
// lanes 4k .. 4k + 3.  Then one online softmax update, with key k's p read
// from lane 4k for the O += p V products (a V row of the [D][B] tile holds
// the chunk's 16 keys contiguously).
template <typename C, int D>
__device__ __forceinline__ void attend_chunk(const C* kc, const C* vc, int64_t tile, int B,
                                             int off0, int j0, int kend, int lane,
                                             const float (&qv)[D / 64], float& m, float& l,
                                             float (&acc)[D / 64]) {
  constexpr int E = D / 64;
  const C* kr = kc + (tile * B + off0) * D + lane * E;             // K tile [B][D]
  float z[kChunk];
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    float p = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) p = fmaf(qv[e], ldc<C>(kr + i * D + e), p);
    z[i] = p;
  }
  float vv[E][kChunk];                                             // V tile [D][B]
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const C* vr = vc + (tile * D + lane * E + e) * B + off0;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) vv[e][i] = ldc<C>(vr + i);
  }
  float z8[8], z4[4], z2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool hi = lane & 32;
    z8[i] = (hi ? z[i + 8] : z[i]) + __shfl_xor(hi ? z[i] : z[i + 8], 32);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool hi = lane & 16;
    z4[i] = (hi ? z8[i + 4] : z8[i]) + __shfl_xor(hi ? z8[i] : z8[i + 4], 16);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool hi = lane & 8;
    z2[i] = (hi ? z4[i + 2] : z4[i]) + __shfl_xor(hi ? z4[i] : z4[i + 2], 8);
  }
  float zk;
  {
    const bool hi = lane & 4;
    zk = (hi ? z2[1] : z2[0]) + __shfl_xor(hi ? z2[0] : z2[1], 4);
  }
  zk += __shfl_xor(zk, 2);
  zk += __shfl_xor(zk, 1);
  zk = j0 + (lane >> 2) < kend ? zk : -INFINITY;
  float bm = zk;
  bm = fmaxf(bm, __shfl_xor(bm, 4));
  bm = fmaxf(bm, __shfl_xor(bm, 8));
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const float mn = fmaxf(m, bm);                  // finite: key j0 is below kend
  const float alpha = expf(m - mn);               // 0 for a first chunk (m = -inf)
  const float pk = expf(zk - mn);                 // 0 for masked keys
  // the chunk's sum of p: the lanes that differ in bits 5..2 hold each key once
  float ps = pk;
  ps += __shfl_xor(ps, 4);
  ps += __shfl_xor(ps, 8);
  ps += __shfl_xor(ps, 16);
  ps += __shfl_xor(ps, 32);
  l = fmaf(l, alpha, ps);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    const float pi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pk), 4 * i));
    const bool in = j0 + i < kend;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(pi, in ? vv[e][i] : 0.0f, acc[e]);
  }
  m = mn;
}

// C: cache element type (T, or uint8_t E4M3FN codes whose values are scaled
// by k_scale / v_scale: folded into the query scaling and the final divide)

// Prefill rows (cu_seqlens given): one wave per (row, head), four rows of one
// sequence and head per workgroup; the wave attends its row's keys 0..pos in
// 16-key chunks and writes the row.
template <typename T, typename C, int D>
__global__ __launch_bounds__(256) void attn_generic_rows_kernel(AttnArgs a) {
  constexpr int E = D / 64;
  const int s = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + w;
  const int r0 = a.cu_seqlens[s];
  const int n = a.cu_seqlens[s + 1] - r0;
  // a row range outside the packed batch (bad cu_seqlens), a negative row
  // count or more rows than any valid context holds: flag, write no row
  if (r0 < 0 || n < 0 || static_cast<int64_t>(r0) + n > a.num_tokens || n > a.max_context_len) {
    if (row == 0 && lane == 0) report_error(a.err, kErrSequence);
    return;
  }
  if (row >= n) return;                           // wave-uniform
  int c = a.context_lens[s];
  bool bad = c < 1 || c > a.max_context_len;     // contract: 1 <= c <= max_context_len
  if (bad && lane == 0) report_error(a.err, kErrSequence);
  if (bad) c = 0;
  const int pos = c - n + row;
  if (pos < 0 && lane == 0) report_error(a.err, kErrSequence);   // more rows than keys
  bad = bad || pos < 0;
  const int Hkv = a.num_kv_heads, B = a.block_size;
  const int g = h / (a.num_heads / Hkv);
  const bool f8 = sizeof(C) == 1;
  const float qs = a.scale * (f8 ? a.k_scale : 1.0f);
  const int64_t t = static_cast<int64_t>(r0) + row;
  const T* qp = static_cast<const T*>(a.q) + t * a.q_stride + static_cast<int64_t>(h) * D + lane * E;
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
  for (int j0 = 0; j0 <= pos; j0 += kChunk) {     // wave-uniform
    const int blk = bt[j0 / B];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      bad = true;
      if (lane == 0) report_error(a.err, kErrBlock);
      break;
    }
    attend_chunk<C, D>(kc, vc, static_cast<int64_t>(blk) * Hkv + g, B, j0 % B, j0, pos + 1, lane,
                       qv, m, l, acc);
  }
  T* op = static_cast<T*>(a.out) + t * a.out_stride + static_cast<int64_t>(h) * D + lane * E;
  const float inv = bad ? __builtin_nanf("") : (f8 ? a.v_scale : 1.0f) / l;
#pragma unroll
  for (int i = 0; i < E; ++i) op[i] = st<T>(acc[i] * inv);
}

// One row per workgroup: the decode rows (one query row per sequence, no
// cu_seqlens; ROWS false), and prefill rows with long contexts (ROWS: row
// blockIdx.x of sequence blockIdx.z).  The workgroup's sixteen waves take
// the 16-key chunks of the row's keys round robin, each keeping its own
// state; the states (m, l, acc) are merged through LDS at the end
// (o = sum_w acc_w e^(m_w - M) / sum_w l_w e^(m_w - M)).  Sixteen waves, not
// four, so that a small batch (a few sequences x heads workgroups) or a long
// row still has many chunks in flight.
template <typename T, typename C, int D, bool ROWS>
__global__ __launch_bounds__(1024) void attn_generic_wide_kernel(AttnArgs a) {
  constexpr int E = D / 64;
  constexpr int NW = 16;
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ float sm[NW], sl[NW], sacc[NW][D];
  __shared__ int sbad;
  int s, c;
  int64_t t;                                      // the row's token
  bool bad;
  if constexpr (ROWS) {
    s = blockIdx.z;
    const int row = blockIdx.x;
    const int r0 = a.cu_seqlens[s];
    const int n = a.cu_seqlens[s + 1] - r0;
    // as in attn_generic_rows_kernel: a row range outside the batch is
    // flagged once and no row is written
    if (r0 < 0 || n < 0 || static_cast<int64_t>(r0) + n > a.num_tokens || n > a.max_context_len) {
      if (row == 0 && threadIdx.x == 0) report_error(a.err, kErrSequence);
      return;
    }
    if (row >= n) return;                         // the whole workgroup
    c = a.context_lens[s];
    bad = c < 1 || c > a.max_context_len;
    if (bad && threadIdx.x == 0) report_error(a.err, kErrSequence);
    const int pos = (bad ? 0 : c) - n + row;
    if (pos < 0 && threadIdx.x == 0) report_error(a.err, kErrSequence);   // more rows than keys
    bad = bad || pos < 0;
    c = bad ? 0 : pos + 1;                        // the row's keys
    t = static_cast<int64_t>(r0) + row;
  } else {
    s = blockIdx.x;
    c = a.context_lens[s];
    bad = c < 1 || c > a.max_context_len;         // contract: 1 <= c <= max_context_len
    if (bad && threadIdx.x == 0) report_error(a.err, kErrSequence);
    if (bad) c = 0;
    t = s;
  }
  if (threadIdx.x == 0) sbad = 0;
  const int Hkv = a.num_kv_heads, B = a.block_size;
  const int g = h / (a.num_heads / Hkv);
  const bool f8 = sizeof(C) == 1;
  const float qs = a.scale * (f8 ? a.k_scale : 1.0f);
  const T* qp = static_cast<const T*>(a.q) + t * a.q_stride + static_cast<int64_t>(h) * D + lane * E;
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
  for (int j0 = w * kChunk; j0 < c; j0 += NW * kChunk) {   // wave-uniform
    const int blk = bt[j0 / B];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      wbad = true;
      break;
    }
    attend_chunk<C, D>(kc, vc, static_cast<int64_t>(blk) * Hkv + g, B, j0 % B, j0, c, lane, qv, m,
                       l, acc);
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
  T* op = static_cast<T*>(a.out) + t * a.out_stride + static_cast<int64_t>(h) * D + lane * E;
#pragma unroll
  for (int i = 0; i < E; ++i) op[i] = st<T>(o[i] * inv);
}

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream) {
  // Prefill rows: a wave per row, or a workgroup per row where every row has
  // a long context (at least kWideKeys keys and four times the longest
  // chunk: a chunk after a long prefix), so that a row's chunks are spread
  // over sixteen waves instead of walked by one.
  constexpr int kWideKeys = 2048;
  const bool wide = a.max_context_len >= kWideKeys && a.max_context_len >= 4 * a.max_query_len;
  const dim3 grid((a.max_query_len + 3) / 4, a.num_heads, a.num_seqs);   // prefill, wave per row
  const dim3 wgrid(a.max_query_len, a.num_heads, a.num_seqs);            // prefill, workgroup per row
  const dim3 dgrid(a.num_seqs, a.num_heads);                             // decode rows
#define QW_GEN(T, C, D)                                                                      \
  do {                                                                                       \
    if (!a.cu_seqlens)                                                                       \
      hipLaunchKernelGGL((attn_generic_wide_kernel<T, C, D, false>), dgrid, dim3(1024), 0,   \
                         stream, a);                                                         \
    else if (wide)                                                                           \
      hipLaunchKernelGGL((attn_generic_wide_kernel<T, C, D, true>), wgrid, dim3(1024), 0,    \
                         stream, a);                                                         \
    else                                                                                     \
      hipLaunchKernelGGL((attn_generic_rows_kernel<T, C, D>), grid, dim3(256), 0, stream, a); \
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
