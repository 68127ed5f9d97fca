/*
 * qwen2_attn.h -- C ABI of the paged GQA attention library (libqwen2attn.so)
 * for one AMD MI355X (gfx950).
 *
 * What it computes: the attention core of a Qwen2 decoder layer as the
 * reference pages describe it running in vLLM.
 *   - The fused QKV projection output is split by columns into q, k, v
 *     ("Qwen2大模型架构解析与vLLM优化实践", §2.2 QKVParallelLinear; §4.3
 *     packed_modules_mapping q_proj/k_proj/v_proj -> qkv_proj).
 *   - q and k are rotated with rotary position embedding over the whole head
 *     dimension with base rope_theta (same page, §2.2 get_rope(head_dim,
 *     rotary_dim=head_dim, max_position, base=rope_theta); "Qwen2 模型结构代码详解",
 *     §2: rope_theta 1e6).  Pairing is NeoX (element i with i + d/2).
 *   - k and v are written into a KV cache cut into fixed-size blocks handed
 *     out like OS pages ("vLLM 部署 Qwen", §2.1 PagedAttention).
 *   - Causal grouped-query attention: query head h reads KV head
 *     h / (num_heads / num_kv_heads) ("Qwen2 模型结构代码详解", §2: 28:4, seven
 *     q heads per KV group), scores scaled by head_dim^-0.5 (same section),
 *     for packed variable-length prefill ("Qwen 开源工程笔记", §3 flash-attn
 *     varlen) and single-token paged decode ("vLLM 部署 Qwen", §2.1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every array argument is a DEVICE pointer unless the comment says
 *   HOST.  The caller owns all memory; the library allocates nothing, keeps
 *   no pointer after returning and holds no global mutable state except a
 *   thread-local error string and the per-GPU scratch array of
 *   qwen2_attn_decode_paged_noalloc.  Entry points are thread-safe (that one
 *   with the restriction it states).
 * Streams: every call enqueues its kernels on `stream` (0 = the null stream)
 *   and returns without synchronising.
 * dtype: QW_BF16 (bfloat16 storage, fp32 arithmetic) or QW_F32.  q, k, v,
 *   q_out, out and both caches share the one dtype.
 * Rows: a "row" is one token.  Within a row the heads are contiguous, each
 *   head_dim elements long.  *_row_stride is the distance between rows in
 *   ELEMENTS (not bytes); it must be >= the row's width and keep every row
 *   16-byte aligned.  Base pointers must be 16-byte aligned.
 * Cache layout (both caches hold num_blocks blocks of block_size tokens):
 *   k_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *   v_cache [num_blocks][num_kv_heads][head_dim][block_size]
 *   A token at logical position p of sequence s lives in physical block
 *   block_tables[s][p / block_size] at offset p % block_size; its slot is
 *   block * block_size + offset.
 * Supported shapes: head_dim 64 or 128, block_size 16, 32 or 64 tokens,
 *   num_heads a multiple of num_kv_heads, group num_heads/num_kv_heads <= 16.
 *   ("Qwen2大模型架构解析与vLLM优化实践", §5.2 configures 64-token cache
 *   blocks; "vLLM 部署 Qwen", §5.1 names a 16-token default raised to 32.
 *   The matrix-core kernels read every size as 16-token blocks.)
 * Errors: host-side validation runs before any launch.  A failing call
 *   returns a nonzero qw_status, launches nothing and records a message for
 *   qwen2_last_error().  Zero-size work returns QW_OK without a launch.
 *   A HIP launch failure returns QW_ERR_HIP.
 * Device metadata contract (device data the host does not read): positions
 *   in [0, max_position); slots in [-1, num_blocks*block_size) with no slot
 *   named twice in one call; block ids of the first ceil(c/B) table entries
 *   in [0, num_blocks); 1 <= context_lens[s] <= max_context_len; query rows
 *   of a sequence sit at positions c - n .. c - 1.  Kernels bounds-check
 *   this metadata and never access memory out of bounds for it: a token
 *   with an out-of-range position writes no K/V and a NaN q_out row; one
 *   with an out-of-range slot writes no K/V (q_out as usual); a sequence
 *   with an out-of-range block id or context length (or more rows than
 *   keys) produces NaN outputs; a prefill sequence whose rows lie outside
 *   the packed batch or number more than max_context_len writes no rows.
 *   Each case also sets a flag in the GPU's device error word
 *   (qwen2_device_errors).  qwen2_check_metadata_host() verifies the whole
 *   contract on host copies.
 * Order per layer step: qwen2_rope_cache_write, then qwen2_attn_prefill_varlen
 *   and/or qwen2_attn_decode_paged, on the same stream.
 */
#ifndef QWEN2_ATTN_H
#define QWEN2_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The entry points below are the library's only exported symbols (it is
 * built with hidden default visibility). */
#pragma GCC visibility push(default)

typedef enum {
  QW_OK = 0,
  QW_ERR_NULL = 1,         /* a required pointer is NULL */
  QW_ERR_SHAPE = 2,        /* inconsistent sizes or strides */
  QW_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head_dim, block_size, dtype, group) */
  QW_ERR_ALIGN = 4,        /* base pointer or row stride breaks 16-byte alignment */
  QW_ERR_WORKSPACE = 5,    /* workspace missing or too small */
  QW_ERR_METADATA = 6,     /* qwen2_check_metadata_host found a violation */
  QW_ERR_HIP = 7           /* a HIP runtime call or launch failed */
} qw_status;

typedef enum { QW_F32 = 0, QW_BF16 = 1 } qw_dtype;

/*
 * Fill the rotary table: for p < max_position, i < rotary_dim/2,
 *   cos_sin[p][i]                = cos(p * f_i)
 *   cos_sin[p][rotary_dim/2 + i] = sin(p * f_i),  f_i = rope_theta^(-2i/rotary_dim)
 * computed and stored in float64 on the device (the angle is never formed
 * in float32, which at p ~ 32767 would be off by ~1e-3 rad).
 * "Qwen2大模型架构解析与vLLM优化实践", §2.2 (get_rope(..., max_position, base));
 * "Qwen2 模型结构代码详解", §3 (max_model_len becomes max_position).
 * cos_sin: device, float64 [max_position][rotary_dim], written.
 * Requires max_position >= 1, rotary_dim even in [2, 256], rope_theta > 0.
 * Call once per (theta, rotary_dim, max_position); the table is read-only after.
 */
int qwen2_rope_table_init(double* cos_sin, int max_position, int rotary_dim,
                          double rope_theta, hipStream_t stream);

/*
 * Dynamic-NTK rope scaling: the table for a context longer than the model's
 * original window.  It has L = qwen2_rope_dynamic_ntk_positions(original,
 * factor) = floor(factor * original_max_position) rows and is the table of
 * qwen2_rope_table_init with the base
 *   rope_theta * (factor * L / original_max_position - (factor - 1))^(d / (d - 2))
 * (d = rotary_dim; the base is formed in float64 on the host): the fastest
 * frequency is unchanged and the slowest turns factor^2 - factor + 1 times
 * slower.  Every other call takes the table (and max_position = L) as usual.
 * "Qwen2大模型架构解析与vLLM优化实践", §7.1 (rope_scaling {"type": "dynamic",
 * "factor", "original_max_position"} raising the RoPE base); "Qwen2 模型结构
 * 代码详解", §3 (rope_scaling handed to get_rope past 32768 positions).
 * cos_sin: device, float64 [L][rotary_dim], written.  Requires
 * original_max_position >= 1, factor >= 1, rotary_dim even in [4, 256],
 * rope_theta > 0.  qwen2_rope_dynamic_ntk_positions returns -1 for invalid
 * arguments.
 */
int qwen2_rope_dynamic_ntk_positions(int original_max_position, double factor);
int qwen2_rope_table_init_dynamic_ntk(double* cos_sin, int original_max_position, double factor,
                                      int rotary_dim, double rope_theta, hipStream_t stream);

/*
 * Rotate q and k of num_tokens tokens and write k, v into the paged cache.
 *   q  [T][num_heads][head_dim]     (q_row_stride elements between tokens)
 *   k  [T][num_kv_heads][head_dim]  (k_row_stride)
 *   v  [T][num_kv_heads][head_dim]  (v_row_stride)
 * q, k, v are typically column views of one fused QKV tensor
 * [T][(H + 2 Hkv) * d] (row stride (H + 2 Hkv) * d for all three).
 * For token t at position p = positions[t], every q and k head is rotated
 * (NeoX pairs (i, i + d/2), angle from cos_sin row p):
 *   y_i = x_i cos - x_{i+d/2} sin,   y_{i+d/2} = x_{i+d/2} cos + x_i sin
 * in float64 (table included) and rounded once, to nearest even, to the
 * storage dtype: stored q/k are the correctly rounded rotation.  Rotated q goes to
 * q_out [T][num_heads][head_dim] (q_out_row_stride; q_out may equal q for
 * an in-place update, any other overlap is undefined).  If slot_mapping[t]
 * >= 0, rotated k goes to k_cache[slot/B][g][slot%B][:] and v is copied bit
 * for bit to v_cache[slot/B][g][:][slot%B]; slot -1 writes nothing.  Slots
 * not named are left untouched.
 * cos_sin: table from qwen2_rope_table_init with rotary_dim == head_dim and
 * max_position rows (max_position * head_dim doubles are readable).  positions, slot_mapping: device int32 [T].
 * "vLLM 部署 Qwen", §2.1 (paged KV cache); "Qwen2大模型架构解析与vLLM优化实践",
 * §7.3 (RoPE as one fused kernel).
 */
int qwen2_rope_cache_write(const void* q, int64_t q_row_stride,
                           void* q_out, int64_t q_out_row_stride,
                           const void* k, int64_t k_row_stride,
                           const void* v, int64_t v_row_stride,
                           const int32_t* positions, const int32_t* slot_mapping,
                           const double* cos_sin, int max_position,
                           void* k_cache, void* v_cache, int num_blocks,
                           int num_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int dtype, hipStream_t stream);

/*
 * Causal GQA attention for packed variable-length query rows (prefill and
 * chunked prefill) over the paged cache.
 *   q   [num_tokens][num_heads][head_dim], already rotated (q_row_stride)
 *   out [num_tokens][num_heads][head_dim], written (out_row_stride)
 *   cu_seqlens_q [num_seqs + 1]: sequence s owns rows cu[s] .. cu[s+1]-1,
 *     cu[0] = 0, cu[num_seqs] <= num_tokens; rows outside every sequence are
 *     not written.
 *   context_lens [num_seqs]: keys of sequence s, the new rows included
 *     (c >= n = cu[s+1] - cu[s]); row i sits at position c - n + i and
 *     attends to keys 0 .. c - n + i.
 *   block_tables [num_seqs][max_blocks_per_seq] int32.
 * max_query_len >= every n (sizes the grid), max_context_len >= every c.
 * scale is the softmax scaling, normally head_dim^-0.5.  Scores and softmax
 * are float32; bf16 uses matrix-core (MFMA) products with fp32 accumulation.
 * The cache must already hold every key the rows attend to (call
 * qwen2_rope_cache_write for the new tokens first).
 * "Qwen 开源工程笔记", §3 (varlen packed prefill); "Qwen2大模型架构解析与vLLM
 * 优化实践", §7.3 (causal mask).
 */
int qwen2_attn_prefill_varlen(const void* q, int64_t q_row_stride,
                              const void* k_cache, const void* v_cache, int num_blocks,
                              const int32_t* cu_seqlens_q, const int32_t* context_lens,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              void* out, int64_t out_row_stride,
                              int num_seqs, int num_tokens, int max_query_len,
                              int max_context_len, int num_heads, int num_kv_heads,
                              int head_dim, int block_size, float scale, int dtype,
                              hipStream_t stream);

/*
 * Bytes of device workspace qwen2_attn_decode_paged needs for these sizes
 * (0 when it needs none).  The same arguments must be passed to the decode
 * call.  Returns (size_t)-1 for unsupported or invalid sizes.
 */
size_t qwen2_attn_decode_workspace_size(int num_seqs, int max_context_len, int num_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int dtype);

/*
 * Single-token paged decode: query row s of q [num_seqs][num_heads][head_dim]
 * (q_row_stride) sits at position context_lens[s] - 1 and attends to all
 * context_lens[s] keys of sequence s (its own key included: write it with
 * qwen2_rope_cache_write first).  out [num_seqs][num_heads][head_dim]
 * (out_row_stride) is written.  The batch's (sequence, KV head, block)
 * units are spread evenly over the GPU: a sequence may be cut into pieces
 * whose partial softmax states are merged exactly (log-sum-exp, in a fixed
 * order, so results are bitwise reproducible) by the workgroup that
 * finishes a sequence's last piece, inside the same kernel; workspace
 * (device, 16-byte aligned, workspace_bytes >=
 * qwen2_attn_decode_workspace_size(...)) holds a work counter, per-range
 * arrival counters and those partial states and is scratch: its contents
 * on entry do not matter (a small launch before the kernel zeroes the
 * counters).
 * Calls that share one workspace must not overlap.
 * "vLLM 部署 Qwen", §2.1 and §4.1 (paged KV access dominates decode).
 */
int qwen2_attn_decode_paged(const void* q, int64_t q_row_stride,
                            const void* k_cache, const void* v_cache, int num_blocks,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens,
                            void* out, int64_t out_row_stride,
                            void* workspace, size_t workspace_bytes,
                            int num_seqs, int max_context_len, int num_heads,
                            int num_kv_heads, int head_dim, int block_size, float scale,
                            int dtype, hipStream_t stream);

/*
 * qwen2_attn_decode_paged_noalloc: qwen2_attn_decode_paged without a
 * workspace argument, for callers that cannot allocate device memory at the
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, kernels and results as
 * qwen2_attn_decode_paged (bitwise equal outputs); the workspace is a
 * static device array of QWEN2_DECODE_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, resolved on the first call on each device (the
 * calling thread's current device, which must be the stream's) and held
 * until the process ends.  The call itself allocates nothing.  The kernels
 * reset the array's counters at the start of every call, so stale contents
 * from an earlier call never matter; but every call on one GPU shares that
 * GPU's array, so calls that overlap in time on one GPU (different streams,
 * or host threads) race and must not be issued.  A decode whose workspace
 * (qwen2_attn_decode_workspace_size) would exceed the array returns
 * QW_ERR_WORKSPACE without launching; every bf16 head_dim-128 decode with
 * group <= 8 fits (at most 1024 ranges of partial states).
 */
#define QWEN2_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)9 << 20)
int qwen2_attn_decode_paged_noalloc(const void* q, int64_t q_row_stride,
                                    const void* k_cache, const void* v_cache, int num_blocks,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens,
                                    void* out, int64_t out_row_stride,
                                    int num_seqs, int max_context_len, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, float scale,
                                    int dtype, hipStream_t stream);

/*
 * FP8 KV cache.  The three calls below are the ones above with a cache of
 * one-byte E4M3FN codes (OCP FP8: sign, 4 exponent bits with bias 7, 3
 * mantissa bits; largest finite value 448; no infinity; S.1111.111 is NaN)
 * and one scale per tensor: a cached key is k_scale * value(code), a cached
 * value v_scale * value(code).  Layouts are unchanged ([num_blocks][Hkv][B][d]
 * and [num_blocks][Hkv][d][B]), one byte per element, so a (block, KV head)
 * tile is 2 KiB at head_dim 128.  q, k, v and out keep `dtype` (bf16 or
 * f32).  k_scale, v_scale must be finite and > 0 (else QW_ERR_SHAPE).
 * "Qwen2大模型架构解析与vLLM优化实践", §4.1-4.2 (FP8 / INT8 KV-cache
 * quantization, per-layer cache scale parameters) and §6.3 (the E4M3FN
 * format).
 *
 * qwen2_rope_cache_write_fp8: as qwen2_rope_cache_write, except that the
 * cache receives code(rot(k) / k_scale) and code(v / v_scale): the exact
 * float64 rotation (or the value) divided by the scale, rounded once to the
 * nearest code (ties to even) and saturated to +-448.  q_out is written as
 * in qwen2_rope_cache_write.
 */
int qwen2_rope_cache_write_fp8(const void* q, int64_t q_row_stride,
                               void* q_out, int64_t q_out_row_stride,
                               const void* k, int64_t k_row_stride,
                               const void* v, int64_t v_row_stride,
                               const int32_t* positions, const int32_t* slot_mapping,
                               const double* cos_sin, int max_position,
                               void* k_cache, void* v_cache, int num_blocks,
                               int num_tokens, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int dtype,
                               float k_scale, float v_scale, hipStream_t stream);

/*
 * qwen2_attn_prefill_varlen_fp8: as qwen2_attn_prefill_varlen over an FP8
 * cache (keys and values read as scale * value(code)).
 */
int qwen2_attn_prefill_varlen_fp8(const void* q, int64_t q_row_stride,
                                  const void* k_cache, const void* v_cache, int num_blocks,
                                  const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  void* out, int64_t out_row_stride,
                                  int num_seqs, int num_tokens, int max_query_len,
                                  int max_context_len, int num_heads, int num_kv_heads,
                                  int head_dim, int block_size, float scale, int dtype,
                                  float k_scale, float v_scale, hipStream_t stream);

/*
 * qwen2_attn_decode_paged_fp8: as qwen2_attn_decode_paged over an FP8 cache;
 * the workspace is sized by qwen2_attn_decode_workspace_size with the same
 * arguments (it does not depend on the cache format).
 */
int qwen2_attn_decode_paged_fp8(const void* q, int64_t q_row_stride,
                                const void* k_cache, const void* v_cache, int num_blocks,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens,
                                void* out, int64_t out_row_stride,
                                void* workspace, size_t workspace_bytes,
                                int num_seqs, int max_context_len, int num_heads,
                                int num_kv_heads, int head_dim, int block_size, float scale,
                                int dtype, float k_scale, float v_scale, hipStream_t stream);

/*
 * Qwen3 q/k norm.  As qwen2_rope_cache_write (resp. _fp8), with every q and k
 * head RMS-normalised over head_dim before the rotation:
 *   x <- x / sqrt(mean_i(x_i^2) + rms_eps) * w     (w = q_norm_weight or
 *   k_norm_weight, device [head_dim] of `dtype`, 16-byte aligned)
 * computed in float64 together with the rotation and rounded once (FP8: the
 * cache code of the normalised, rotated k divided by k_scale).  v is not
 * normalised.  rms_eps must be finite and >= 0 (Qwen3: 1e-6).
 * "nano-vllm: Qwen3 骨架", §5 (the q_norm / k_norm RMSNorm modules of the
 * attention) and §3.2 (rms_norm_eps).
 */
int qwen3_rope_cache_write(const void* q, int64_t q_row_stride,
                           void* q_out, int64_t q_out_row_stride,
                           const void* k, int64_t k_row_stride,
                           const void* v, int64_t v_row_stride,
                           const int32_t* positions, const int32_t* slot_mapping,
                           const double* cos_sin, int max_position,
                           void* k_cache, void* v_cache, int num_blocks,
                           int num_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int dtype,
                           const void* q_norm_weight, const void* k_norm_weight, double rms_eps,
                           hipStream_t stream);

int qwen3_rope_cache_write_fp8(const void* q, int64_t q_row_stride,
                               void* q_out, int64_t q_out_row_stride,
                               const void* k, int64_t k_row_stride,
                               const void* v, int64_t v_row_stride,
                               const int32_t* positions, const int32_t* slot_mapping,
                               const double* cos_sin, int max_position,
                               void* k_cache, void* v_cache, int num_blocks,
                               int num_tokens, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int dtype,
                               const void* q_norm_weight, const void* k_norm_weight,
                               double rms_eps, float k_scale, float v_scale, hipStream_t stream);

/*
 * Shared-prefix (cascade) decode.  With prefix caching, sequences that start
 * with the same prompt hold the same physical KV blocks for it ("Qwen2 模型
 * 结构代码详解", §3: enable_prefix_caching makes the attention layer reuse the
 * KV blocks of an identical prefix; §4 shows the reuse).  These calls compute
 * exactly what qwen2_attn_decode_paged (resp. _fp8) computes -- softmax
 * attention of each sequence's query over all keys of its block table -- but
 * read each group's shared prefix blocks from HBM once for the whole group
 * instead of once per member: the group's (member, query head) pairs are
 * attended to the prefix together (16 per MFMA tile, in chunks of blocks),
 * every member's private keys after the prefix by the decode's stream
 * kernel, and the partial softmax states merged exactly.
 *
 * Prefix groups (DEVICE int32 arrays): group p's members are the sequences
 * prefix_seqs[prefix_indptr[p] .. prefix_indptr[p + 1]) (indices into this
 * call's batch); its prefix is the first prefix_lens[p] tokens of each
 * member, a multiple of block_size, which every member's block table names
 * with the same block ids (the group's ids are read from its first member's
 * table).  Contract (not checked on the device; qwen2_check_prefix_groups_host
 * checks it on host copies): prefix_indptr rises from 0 to num_prefix_members;
 * each member appears once; 0 < prefix_lens[p] <= max_prefix_len; every
 * member's context exceeds its prefix; members share the prefix block ids.
 * A group whose length is not a positive multiple of block_size up to
 * max_prefix_len, or whose first member is out of range or has no key
 * after the prefix, is not used, and a member with no key after its prefix
 * is decoded plainly: those sequences' results stay exact.  Members that do
 * not hold the ids of the first member's table, or a sequence listed in two
 * groups, give wrong outputs for those sequences (never out-of-bounds
 * accesses).
 *
 * num_prefixes, num_prefix_members, max_prefix_len: HOST ints (>= 0).  With
 * no group, no member or max_prefix_len < block_size, and for shapes other
 * than bf16 / head_dim 128 / G <= 8, the call is the plain
 * decode.  Workspace: qwen2_attn_decode_cascade_workspace_size(...) bytes,
 * scratch as for the plain decode (it holds, besides the decode's part, the
 * prefix chunk states: about 16 chunks x num_seqs x num_heads x 520 bytes).
 * Calls that share one workspace must not overlap.  Errors as for
 * qwen2_attn_decode_paged, plus QW_ERR_NULL for NULL group arrays with
 * num_prefixes > 0 and QW_ERR_SHAPE for negative counts or a prefix-level
 * grid beyond 2^31 - 2 workgroups.
 */
/*
 * Whether the shared-prefix (cascade) decode is expected to beat the plain
 * decode for a batch with these prefix groups: 1 when the prefix KV bytes it
 * saves, (num_prefix_members - num_prefixes) * max_prefix_len * num_kv_heads
 * * 2 * head_dim * element bytes (1 with cache_fp8, else 2), reach 96 MiB,
 * else 0.  The cascade pays one more launch and a prefix pass before the
 * private keys; on this GPU it lost ~3 us with 49 MB saved (48 members of a
 * 1024-token prefix over 2 KV heads) and gained ~38 us with 503 MB saved
 * (4 groups of 16 over 4096 tokens and 4 KV heads), a break-even near
 * 80 MB.  Callers that leave the choice to the library call the cascade
 * entry point only when this returns 1 (the results agree either way).
 * Pure host function; returns 0 for negative or zero counts.
 */
int qwen2_attn_decode_cascade_worthwhile(int num_prefixes, int num_prefix_members,
                                         int max_prefix_len, int num_kv_heads, int head_dim,
                                         int cache_fp8);

size_t qwen2_attn_decode_cascade_workspace_size(int num_seqs, int max_context_len,
                                                int max_prefix_len, int num_prefixes,
                                                int num_prefix_members, int num_heads,
                                                int num_kv_heads, int head_dim, int block_size,
                                                int dtype);

int qwen2_attn_decode_paged_cascade(const void* q, int64_t q_row_stride,
                                    const void* k_cache, const void* v_cache, int num_blocks,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens,
                                    const int32_t* prefix_indptr, const int32_t* prefix_seqs,
                                    const int32_t* prefix_lens, int num_prefixes,
                                    int num_prefix_members, int max_prefix_len,
                                    void* out, int64_t out_row_stride,
                                    void* workspace, size_t workspace_bytes,
                                    int num_seqs, int max_context_len, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, float scale,
                                    int dtype, hipStream_t stream);

int qwen2_attn_decode_paged_cascade_fp8(const void* q, int64_t q_row_stride,
                                        const void* k_cache, const void* v_cache, int num_blocks,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens,
                                        const int32_t* prefix_indptr, const int32_t* prefix_seqs,
                                        const int32_t* prefix_lens, int num_prefixes,
                                        int num_prefix_members, int max_prefix_len,
                                        void* out, int64_t out_row_stride,
                                        void* workspace, size_t workspace_bytes,
                                        int num_seqs, int max_context_len, int num_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        float scale, int dtype, float k_scale, float v_scale,
                                        hipStream_t stream);

/*
 * Verify the prefix-group contract of the cascade calls on HOST copies
 * (prefix_indptr [num_prefixes + 1], prefix_seqs [num_prefix_members],
 * prefix_lens [num_prefixes], context_lens [num_seqs], block_tables
 * [num_seqs][max_blocks_per_seq]).  Returns QW_OK or QW_ERR_METADATA (first
 * violation in qwen2_last_error()).  No HIP call is made.
 */
int qwen2_check_prefix_groups_host(const int32_t* prefix_indptr, const int32_t* prefix_seqs,
                                   const int32_t* prefix_lens, int num_prefixes,
                                   int num_prefix_members, int max_prefix_len,
                                   const int32_t* context_lens, const int32_t* block_tables,
                                   int num_seqs, int max_blocks_per_seq, int block_size);

/*
 * Verify the device-metadata contract on HOST copies (tests, debugging).
 * positions, slot_mapping: HOST int32 [num_tokens] (either may be NULL to
 * skip it).  cu_seqlens_q: HOST int32 [num_seqs + 1], or NULL for a decode
 * batch (row s = sequence s).  context_lens: HOST int32 [num_seqs].
 * block_tables: HOST int32 [num_seqs][max_blocks_per_seq].
 * Checks: position/slot ranges, no duplicate slot, cu monotone from 0,
 * 1 <= n <= c <= max_context_len, n <= max_query_len (when > 0), used
 * block ids in range, positions[t] == c - n + i for the rows of each
 * sequence, and slot_mapping[t] naming the block-table slot of that
 * position.  Returns QW_OK or QW_ERR_METADATA (first violation in
 * qwen2_last_error()).  No HIP call is made.
 */
int qwen2_check_metadata_host(const int32_t* positions, const int32_t* slot_mapping,
                              int num_tokens, const int32_t* cu_seqlens_q,
                              const int32_t* context_lens, const int32_t* block_tables,
                              int num_seqs, int max_blocks_per_seq, int num_blocks,
                              int block_size, int max_position, int max_context_len,
                              int max_query_len);

/*
 * Device error word (debugging aid).  Each GPU holds one 32-bit word inside
 * the library, zero when the library loads.  When a kernel meets device
 * metadata outside the contract above, besides producing NaN outputs or
 * skipping the write it ORs a flag into the word of the GPU it runs on:
 */
#define QW_DEVICE_ERR_POSITION 1u  /* a position outside [0, max_position) */
#define QW_DEVICE_ERR_SLOT 2u      /* a slot outside [-1, num_blocks * block_size) */
#define QW_DEVICE_ERR_BLOCK 4u     /* a block id the attention reads outside [0, num_blocks) */
#define QW_DEVICE_ERR_SEQUENCE 8u  /* a context length outside [1, max_context_len], more rows than
                                      keys, or a row range outside the packed batch (a negative
                                      row count included) */
/*
 * qwen2_device_errors reads the current device's word into *flags (HOST
 * pointer) and, if clear != 0, resets it to zero.  It synchronises with the
 * device (a blocking copy), so it is for tests and debugging, not for a hot
 * path or graph capture.  The word gathers the flags of every call on that
 * GPU since it was last cleared, from any thread or stream.  Returns QW_OK,
 * QW_ERR_NULL for a NULL flags pointer, or QW_ERR_HIP.
 */
int qwen2_device_errors(unsigned int* flags, int clear);

/* Static text for a qw_status value. */
const char* qwen2_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* qwen2_last_error(void);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* QWEN2_ATTN_H */
