// Internal launcher interface between the C-ABI layer (qwen2_attn_api.cpp)
// and the kernel translation units.  Arguments have been validated by the
// caller; launchers only pick a kernel variant and launch it.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qw {

enum Dtype { kF32 = 0, kBF16 = 1 };

struct RopeWriteArgs {
  const void* q; int64_t q_stride;
  void* q_out; int64_t q_out_stride;
  const void* k; int64_t k_stride;
  const void* v; int64_t v_stride;
  const int32_t* positions;
  const int32_t* slots;
  const double* cos_sin; int max_position;
  void* k_cache; void* v_cache; int num_blocks;
  int num_tokens, num_heads, num_kv_heads, head_dim, block_size;
  int dtype;
  int cache_fp8;                 // caches hold E4M3FN codes of value / scale
  float k_scale, v_scale;
  const void* q_norm_w;          // Qwen3 q/k RMSNorm weights [head_dim] (dtype), or null
  const void* k_norm_w;
  double rms_eps;
  unsigned* err;                 // the GPU's device error word (may be null)
};

struct AttnArgs {
  const void* q; int64_t q_stride;
  const void* k_cache; const void* v_cache; int num_blocks;
  const int32_t* cu_seqlens;     // nullptr: one query row per sequence (decode)
  const int32_t* context_lens;
  const int32_t* block_tables; int max_blocks;
  void* out; int64_t out_stride;
  int num_seqs, num_tokens, max_query_len, max_context_len;
  int num_heads, num_kv_heads, head_dim, block_size;
  float scale;
  int dtype;
  void* workspace; size_t workspace_bytes;
  int cache_fp8;                 // caches hold E4M3FN codes; value = code * scale
  float k_scale, v_scale;
  unsigned* err;                 // the GPU's device error word (may be null)
};

// decode plan: which kernel runs and how much workspace it needs
struct DecodePlan {
  bool fast;          // stream-split bf16 kernel (else the generic kernel)
  int num_ranges;     // workgroups (ranges of work units) of the stream kernel
  size_t ws_bytes;
};

DecodePlan plan_decode(int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, int dtype, int cache_fp8);

// shared-prefix cascade decode: the prefix groups (device arrays) and the
// plan (the private level's decode plan, chunking of the prefix level,
// workspace layout after the decode's own part)
struct CascadeMeta {
  const int32_t* indptr;   // [num_prefixes + 1]
  const int32_t* seqs;     // [num_members]
  const int32_t* lens;     // [num_prefixes], tokens
  int num_prefixes, num_members, max_prefix_len;
};
struct CascadePlan {
  DecodePlan dec;
  bool active;             // else the plain decode runs (same result)
  int chunk_blocks, max_chunks, col_wgs;
  int64_t tasks;           // prefix-level workgroups (plus one for the set-up)
  size_t cas_off, pre_ml_off, pre_acc_off, ws_bytes;
};
CascadePlan plan_cascade(int num_seqs, int max_context_len, int max_prefix_len, int num_members,
                         int num_prefixes, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int dtype, int cache_fp8);
hipError_t launch_decode_cascade(const AttnArgs& a, const CascadeMeta& m, const CascadePlan& p,
                                 hipStream_t stream);

hipError_t launch_rope_table(double* tab, int max_position, int rotary_dim, double theta,
                             hipStream_t stream);
hipError_t launch_rope_cache_write(const RopeWriteArgs& a, hipStream_t stream);
hipError_t launch_decode(const AttnArgs& a, const DecodePlan& plan, hipStream_t stream);
hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream);

}  // namespace qw
