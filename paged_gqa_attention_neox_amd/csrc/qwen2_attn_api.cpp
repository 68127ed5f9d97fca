// C ABI of libqwen2attn.so: argument validation, status codes, dispatch to
// the kernel launchers.  Declared (and documented) in include/qwen2_attn.h.
// No allocation; retained state: the thread-local error message, and per GPU
// the device error word and the no-alloc decode's static scratch.
#include "../../include/qwen2_attn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"

#include <cmath>

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return QW_OK;
}

// Device error word, one per GPU (zero when the library loads): the kernels
// OR QW_DEVICE_ERR_* flags into it when they meet metadata outside its
// contract.  In host code the name is only a stand-in for the symbol; the
// kernels get the address hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ unsigned int device_errors;

constexpr int kMaxDevs = 64;
std::mutex g_errword_mu;
unsigned* g_errword_ptr[kMaxDevs] = {};

int current_error_word(unsigned** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QW_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevs) return fail(QW_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevs);
  std::lock_guard<std::mutex> lock(g_errword_mu);
  if (!g_errword_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(device_errors));
    if (e != hipSuccess || !p)
      return fail(QW_ERR_HIP, "hipGetSymbolAddress(device_errors) on device %d failed: %s", dev,
                  hipGetErrorString(e));
    g_errword_ptr[dev] = static_cast<unsigned*>(p);
  }
  *ptr = g_errword_ptr[dev];
  return QW_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == QW_BF16 ? 2 : 4; }

// shared checks of the head layout
int check_heads(int num_heads, int num_kv_heads, int head_dim, int block_size, int dtype) {
  if (dtype != QW_BF16 && dtype != QW_F32) return fail(QW_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(QW_ERR_SHAPE, "num_heads=%d num_kv_heads=%d must be positive", num_heads, num_kv_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(QW_ERR_SHAPE, "num_heads=%d is not a multiple of num_kv_heads=%d", num_heads, num_kv_heads);
  if (num_heads / num_kv_heads > 16)
    return fail(QW_ERR_UNSUPPORTED, "group %d > 16 not supported", num_heads / num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(QW_ERR_UNSUPPORTED, "head_dim=%d not supported (64 or 128)", head_dim);
  if (block_size != 16 && block_size != 32 && block_size != 64)
    return fail(QW_ERR_UNSUPPORTED, "block_size=%d not supported (16, 32 or 64)", block_size);
  return QW_OK;
}

// a [rows][width] view with row stride `stride` (elements)
int check_rows(const char* name, const void* p, int64_t stride, int64_t width, int dtype) {
  if (!p) return fail(QW_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(QW_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (stride < width) return fail(QW_ERR_SHAPE, "%s row stride %lld < row width %lld", name,
                                  static_cast<long long>(stride), static_cast<long long>(width));
  if ((stride * elem_size(dtype)) % 16 != 0)
    return fail(QW_ERR_ALIGN, "%s row stride %lld elements breaks 16-byte alignment", name,
                static_cast<long long>(stride));
  return QW_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(QW_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* qwen2_status_string(int status) {
  switch (status) {
    case QW_OK: return "ok";
    case QW_ERR_NULL: return "null pointer";
    case QW_ERR_SHAPE: return "bad shape or stride";
    case QW_ERR_UNSUPPORTED: return "unsupported configuration";
    case QW_ERR_ALIGN: return "misaligned pointer or stride";
    case QW_ERR_WORKSPACE: return "workspace missing or too small";
    case QW_ERR_METADATA: return "metadata contract violated";
    case QW_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* qwen2_last_error(void) { return g_err; }

int qwen2_device_errors(unsigned int* flags, int clear) {
  if (!flags) return fail(QW_ERR_NULL, "flags is NULL");
  unsigned* word = nullptr;
  const int st = current_error_word(&word);
  if (st) return st;
  hipError_t e = hipMemcpy(flags, word, sizeof(unsigned), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(QW_ERR_HIP, "reading the device error word failed: %s", hipGetErrorString(e));
  if (clear) {
    e = hipMemset(word, 0, sizeof(unsigned));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess)
      return fail(QW_ERR_HIP, "clearing the device error word failed: %s", hipGetErrorString(e));
  }
  return ok();
}

int qwen2_rope_table_init(double* cos_sin, int max_position, int rotary_dim, double rope_theta,
                          hipStream_t stream) {
  if (!cos_sin) return fail(QW_ERR_NULL, "cos_sin is NULL");
  if (max_position < 1) return fail(QW_ERR_SHAPE, "max_position=%d < 1", max_position);
  if (rotary_dim < 2 || rotary_dim > 256 || rotary_dim % 2)
    return fail(QW_ERR_SHAPE, "rotary_dim=%d must be even in [2, 256]", rotary_dim);
  if (!(rope_theta > 0.0)) return fail(QW_ERR_SHAPE, "rope_theta must be > 0");
  return launched(qw::launch_rope_table(cos_sin, max_position, rotary_dim, rope_theta, stream));
}

int qwen2_rope_dynamic_ntk_positions(int original_max_position, double factor) {
  if (original_max_position < 1 || !(factor >= 1.0) || !(factor * original_max_position < 2147483647.0))
    return -1;
  return static_cast<int>(factor * original_max_position);
}

int qwen2_rope_table_init_dynamic_ntk(double* cos_sin, int original_max_position, double factor,
                                      int rotary_dim, double rope_theta, hipStream_t stream) {
  if (!cos_sin) return fail(QW_ERR_NULL, "cos_sin is NULL");
  const int L = qwen2_rope_dynamic_ntk_positions(original_max_position, factor);
  if (L < 1)
    return fail(QW_ERR_SHAPE, "original_max_position=%d and factor=%g give no table",
                original_max_position, factor);
  if (rotary_dim < 4 || rotary_dim > 256 || rotary_dim % 2)
    return fail(QW_ERR_SHAPE, "rotary_dim=%d must be even in [4, 256]", rotary_dim);
  if (!(rope_theta > 0.0)) return fail(QW_ERR_SHAPE, "rope_theta must be > 0");
  // the base grows so that the slowest rotation turns factor L / original -
  // (factor - 1) times slower over the longer table (d / (d - 2) exponent)
  const double d = rotary_dim;
  const double base = rope_theta * std::pow(factor * L / static_cast<double>(original_max_position) -
                                            (factor - 1.0), d / (d - 2.0));
  if (!(base > 0.0) || !(base < 1e300)) return fail(QW_ERR_SHAPE, "scaled rope base out of range");
  return launched(qw::launch_rope_table(cos_sin, L, rotary_dim, base, stream));
}

static int check_fp8_scales(float k_scale, float v_scale) {
  if (!(k_scale > 0.0f) || !(k_scale < 1e30f) || !(v_scale > 0.0f) || !(v_scale < 1e30f))
    return fail(QW_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  return QW_OK;
}

static int rope_write_impl(const void* q, int64_t q_row_stride, void* q_out, int64_t q_out_row_stride,
                           const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                           const int32_t* positions, const int32_t* slot_mapping,
                           const double* cos_sin, int max_position, void* k_cache, void* v_cache,
                           int num_blocks, int num_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int dtype, int cache_fp8, float k_scale,
                           float v_scale, const void* q_norm_w, const void* k_norm_w,
                           double rms_eps, hipStream_t stream) {
  int st = check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st) return st;
  if (cache_fp8 && (st = check_fp8_scales(k_scale, v_scale))) return st;
  if ((q_norm_w != nullptr) != (k_norm_w != nullptr))
    return fail(QW_ERR_NULL, "q_norm_weight and k_norm_weight must both be given");
  if (q_norm_w && (!aligned16(q_norm_w) || !aligned16(k_norm_w)))
    return fail(QW_ERR_ALIGN, "q/k norm weights are not 16-byte aligned");
  if (q_norm_w && !(rms_eps >= 0.0 && rms_eps < 1e300))
    return fail(QW_ERR_SHAPE, "rms_eps must be finite and >= 0");
  if (num_tokens < 0) return fail(QW_ERR_SHAPE, "num_tokens=%d < 0", num_tokens);
  if (num_blocks < 0) return fail(QW_ERR_SHAPE, "num_blocks=%d < 0", num_blocks);
  if (max_position < 1) return fail(QW_ERR_SHAPE, "max_position=%d < 1", max_position);
  if (num_tokens == 0) return ok();
  const int64_t qw = static_cast<int64_t>(num_heads) * head_dim;
  const int64_t kw = static_cast<int64_t>(num_kv_heads) * head_dim;
  if ((st = check_rows("q", q, q_row_stride, qw, dtype))) return st;
  if ((st = check_rows("q_out", q_out, q_out_row_stride, qw, dtype))) return st;
  if ((st = check_rows("k", k, k_row_stride, kw, dtype))) return st;
  if ((st = check_rows("v", v, v_row_stride, kw, dtype))) return st;
  if (q_out != q) {
    // q_out may equal q (in place); any other overlap with the q rows is undefined
    const char* a0 = static_cast<const char*>(q);
    const char* a1 = a0 + ((num_tokens - 1) * q_row_stride + qw) * elem_size(dtype);
    const char* b0 = static_cast<const char*>(q_out);
    const char* b1 = b0 + ((num_tokens - 1) * q_out_row_stride + qw) * elem_size(dtype);
    if (b0 < a1 && a0 < b1)
      return fail(QW_ERR_SHAPE, "q_out overlaps q without being equal to it");
  }
  if (!positions) return fail(QW_ERR_NULL, "positions is NULL");
  if (!slot_mapping) return fail(QW_ERR_NULL, "slot_mapping is NULL");
  if (!cos_sin) return fail(QW_ERR_NULL, "cos_sin is NULL");
  if (!aligned16(cos_sin)) return fail(QW_ERR_ALIGN, "cos_sin is not 16-byte aligned");
  if (num_blocks > 0 && (!k_cache || !v_cache)) return fail(QW_ERR_NULL, "k_cache/v_cache is NULL");
  if (num_blocks > 0 && (!aligned16(k_cache) || !aligned16(v_cache)))
    return fail(QW_ERR_ALIGN, "k_cache/v_cache is not 16-byte aligned");
  qw::RopeWriteArgs a{};
  a.q = q; a.q_stride = q_row_stride;
  a.q_out = q_out; a.q_out_stride = q_out_row_stride;
  a.k = k; a.k_stride = k_row_stride;
  a.v = v; a.v_stride = v_row_stride;
  a.positions = positions; a.slots = slot_mapping;
  a.cos_sin = cos_sin; a.max_position = max_position;
  a.k_cache = k_cache; a.v_cache = v_cache; a.num_blocks = num_blocks;
  a.num_tokens = num_tokens; a.num_heads = num_heads; a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim; a.block_size = block_size; a.dtype = dtype;
  a.cache_fp8 = cache_fp8; a.k_scale = k_scale; a.v_scale = v_scale;
  a.q_norm_w = q_norm_w; a.k_norm_w = k_norm_w; a.rms_eps = rms_eps;
  if ((st = current_error_word(&a.err))) return st;
  return launched(qw::launch_rope_cache_write(a, stream));
}

int qwen2_rope_cache_write(const void* q, int64_t q_row_stride, void* q_out, int64_t q_out_row_stride,
                           const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                           const int32_t* positions, const int32_t* slot_mapping,
                           const double* cos_sin, int max_position, void* k_cache, void* v_cache,
                           int num_blocks, int num_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int dtype, hipStream_t stream) {
  return rope_write_impl(q, q_row_stride, q_out, q_out_row_stride, k, k_row_stride, v, v_row_stride,
                         positions, slot_mapping, cos_sin, max_position, k_cache, v_cache,
                         num_blocks, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                         dtype, 0, 1.0f, 1.0f, nullptr, nullptr, 0.0, stream);
}

int qwen2_rope_cache_write_fp8(const void* q, int64_t q_row_stride, void* q_out,
                               int64_t q_out_row_stride, const void* k, int64_t k_row_stride,
                               const void* v, int64_t v_row_stride, const int32_t* positions,
                               const int32_t* slot_mapping, const double* cos_sin, int max_position,
                               void* k_cache, void* v_cache, int num_blocks, int num_tokens,
                               int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int dtype, float k_scale, float v_scale, hipStream_t stream) {
  return rope_write_impl(q, q_row_stride, q_out, q_out_row_stride, k, k_row_stride, v, v_row_stride,
                         positions, slot_mapping, cos_sin, max_position, k_cache, v_cache,
                         num_blocks, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                         dtype, 1, k_scale, v_scale, nullptr, nullptr, 0.0, stream);
}

int qwen3_rope_cache_write(const void* q, int64_t q_row_stride, void* q_out, int64_t q_out_row_stride,
                           const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                           const int32_t* positions, const int32_t* slot_mapping,
                           const double* cos_sin, int max_position, void* k_cache, void* v_cache,
                           int num_blocks, int num_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int dtype, const void* q_norm_weight,
                           const void* k_norm_weight, double rms_eps, hipStream_t stream) {
  if (!q_norm_weight || !k_norm_weight) return fail(QW_ERR_NULL, "q/k norm weight is NULL");
  return rope_write_impl(q, q_row_stride, q_out, q_out_row_stride, k, k_row_stride, v, v_row_stride,
                         positions, slot_mapping, cos_sin, max_position, k_cache, v_cache,
                         num_blocks, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                         dtype, 0, 1.0f, 1.0f, q_norm_weight, k_norm_weight, rms_eps, stream);
}

int qwen3_rope_cache_write_fp8(const void* q, int64_t q_row_stride, void* q_out,
                               int64_t q_out_row_stride, const void* k, int64_t k_row_stride,
                               const void* v, int64_t v_row_stride, const int32_t* positions,
                               const int32_t* slot_mapping, const double* cos_sin, int max_position,
                               void* k_cache, void* v_cache, int num_blocks, int num_tokens,
                               int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int dtype, const void* q_norm_weight, const void* k_norm_weight,
                               double rms_eps, float k_scale, float v_scale, hipStream_t stream) {
  if (!q_norm_weight || !k_norm_weight) return fail(QW_ERR_NULL, "q/k norm weight is NULL");
  return rope_write_impl(q, q_row_stride, q_out, q_out_row_stride, k, k_row_stride, v, v_row_stride,
                         positions, slot_mapping, cos_sin, max_position, k_cache, v_cache,
                         num_blocks, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                         dtype, 1, k_scale, v_scale, q_norm_weight, k_norm_weight, rms_eps, stream);
}

static int check_attn_common(const void* q, int64_t q_row_stride, const void* k_cache,
                             const void* v_cache, int num_blocks, const int32_t* context_lens,
                             const int32_t* block_tables, int max_blocks_per_seq, const void* out,
                             int64_t out_row_stride, int num_seqs, int max_context_len,
                             int num_heads, int num_kv_heads, int head_dim, int block_size,
                             float scale, int dtype) {
  int st = check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st) return st;
  const int64_t qw = static_cast<int64_t>(num_heads) * head_dim;
  if ((st = check_rows("q", q, q_row_stride, qw, dtype))) return st;
  if ((st = check_rows("out", out, out_row_stride, qw, dtype))) return st;
  if (num_blocks < 1) return fail(QW_ERR_SHAPE, "num_blocks=%d < 1", num_blocks);
  if (!k_cache || !v_cache) return fail(QW_ERR_NULL, "k_cache/v_cache is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(QW_ERR_ALIGN, "k_cache/v_cache is not 16-byte aligned");
  if (!context_lens) return fail(QW_ERR_NULL, "context_lens is NULL");
  if (!block_tables) return fail(QW_ERR_NULL, "block_tables is NULL");
  if (max_context_len < 1) return fail(QW_ERR_SHAPE, "max_context_len=%d < 1", max_context_len);
  if (max_blocks_per_seq < 1 ||
      static_cast<int64_t>(max_blocks_per_seq) * block_size < max_context_len)
    return fail(QW_ERR_SHAPE, "max_blocks_per_seq=%d cannot hold max_context_len=%d",
                max_blocks_per_seq, max_context_len);
  if (!(scale > 0.0f) || !(scale < 1e30f)) return fail(QW_ERR_SHAPE, "scale must be finite and > 0");
  (void)num_seqs;
  return QW_OK;
}

static int prefill_impl(const void* q, int64_t q_row_stride, const void* k_cache,
                        const void* v_cache, int num_blocks, const int32_t* cu_seqlens_q,
                        const int32_t* context_lens, const int32_t* block_tables,
                        int max_blocks_per_seq, void* out, int64_t out_row_stride, int num_seqs,
                        int num_tokens, int max_query_len, int max_context_len, int num_heads,
                        int num_kv_heads, int head_dim, int block_size, float scale, int dtype,
                        int cache_fp8, float k_scale, float v_scale, hipStream_t stream) {
  if (cache_fp8) {
    const int st = check_fp8_scales(k_scale, v_scale);
    if (st) return st;
  }
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0)
    return fail(QW_ERR_SHAPE, "negative size (num_seqs=%d num_tokens=%d max_query_len=%d)",
                num_seqs, num_tokens, max_query_len);
  if (num_seqs > 65535) return fail(QW_ERR_UNSUPPORTED, "num_seqs=%d > 65535", num_seqs);
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) {
    int st = check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype);
    return st ? st : ok();
  }
  int st = check_attn_common(q, q_row_stride, k_cache, v_cache, num_blocks, context_lens,
                             block_tables, max_blocks_per_seq, out, out_row_stride, num_seqs,
                             max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                             scale, dtype);
  if (st) return st;
  if (!cu_seqlens_q) return fail(QW_ERR_NULL, "cu_seqlens_q is NULL");
  if (max_query_len > max_context_len)
    return fail(QW_ERR_SHAPE, "max_query_len=%d > max_context_len=%d", max_query_len, max_context_len);
  qw::AttnArgs a{};
  a.q = q; a.q_stride = q_row_stride;
  a.k_cache = k_cache; a.v_cache = v_cache; a.num_blocks = num_blocks;
  a.cu_seqlens = cu_seqlens_q; a.context_lens = context_lens;
  a.block_tables = block_tables; a.max_blocks = max_blocks_per_seq;
  a.out = out; a.out_stride = out_row_stride;
  a.num_seqs = num_seqs; a.num_tokens = num_tokens;
  a.max_query_len = max_query_len; a.max_context_len = max_context_len;
  a.num_heads = num_heads; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim;
  a.block_size = block_size; a.scale = scale; a.dtype = dtype;
  a.cache_fp8 = cache_fp8; a.k_scale = k_scale; a.v_scale = v_scale;
  if ((st = current_error_word(&a.err))) return st;
  return launched(qw::launch_prefill(a, stream));
}

int qwen2_attn_prefill_varlen(const void* q, int64_t q_row_stride, const void* k_cache,
                              const void* v_cache, int num_blocks, const int32_t* cu_seqlens_q,
                              const int32_t* context_lens, const int32_t* block_tables,
                              int max_blocks_per_seq, void* out, int64_t out_row_stride,
                              int num_seqs, int num_tokens, int max_query_len, int max_context_len,
                              int num_heads, int num_kv_heads, int head_dim, int block_size,
                              float scale, int dtype, hipStream_t stream) {
  return prefill_impl(q, q_row_stride, k_cache, v_cache, num_blocks, cu_seqlens_q, context_lens,
                      block_tables, max_blocks_per_seq, out, out_row_stride, num_seqs, num_tokens,
                      max_query_len, max_context_len, num_heads, num_kv_heads, head_dim,
                      block_size, scale, dtype, 0, 1.0f, 1.0f, stream);
}

int qwen2_attn_prefill_varlen_fp8(const void* q, int64_t q_row_stride, const void* k_cache,
                                  const void* v_cache, int num_blocks, const int32_t* cu_seqlens_q,
                                  const int32_t* context_lens, const int32_t* block_tables,
                                  int max_blocks_per_seq, void* out, int64_t out_row_stride,
                                  int num_seqs, int num_tokens, int max_query_len,
                                  int max_context_len, int num_heads, int num_kv_heads,
                                  int head_dim, int block_size, float scale, int dtype,
                                  float k_scale, float v_scale, hipStream_t stream) {
  return prefill_impl(q, q_row_stride, k_cache, v_cache, num_blocks, cu_seqlens_q, context_lens,
                      block_tables, max_blocks_per_seq, out, out_row_stride, num_seqs, num_tokens,
                      max_query_len, max_context_len, num_heads, num_kv_heads, head_dim,
                      block_size, scale, dtype, 1, k_scale, v_scale, stream);
}

size_t qwen2_attn_decode_workspace_size(int num_seqs, int max_context_len, int num_heads,
                                        int num_kv_heads, int head_dim, int block_size, int dtype) {
  if (num_seqs < 0 || max_context_len < 1) return static_cast<size_t>(-1);
  if (check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype)) return static_cast<size_t>(-1);
  return qw::plan_decode(num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                         dtype, 0).ws_bytes;
}

static qw::AttnArgs decode_args(const void* q, int64_t q_row_stride, const void* k_cache,
                                const void* v_cache, int num_blocks, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* context_lens, void* out,
                                int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                                int num_seqs, int max_context_len, int num_heads,
                                int num_kv_heads, int head_dim, int block_size, float scale,
                                int dtype, int cache_fp8, float k_scale, float v_scale) {
  qw::AttnArgs a{};
  a.q = q; a.q_stride = q_row_stride;
  a.k_cache = k_cache; a.v_cache = v_cache; a.num_blocks = num_blocks;
  a.cu_seqlens = nullptr; a.context_lens = context_lens;
  a.block_tables = block_tables; a.max_blocks = max_blocks_per_seq;
  a.out = out; a.out_stride = out_row_stride;
  a.num_seqs = num_seqs; a.num_tokens = num_seqs; a.max_query_len = 1;
  a.max_context_len = max_context_len;
  a.num_heads = num_heads; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim;
  a.block_size = block_size; a.scale = scale; a.dtype = dtype;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.cache_fp8 = cache_fp8; a.k_scale = k_scale; a.v_scale = v_scale;
  return a;
}

// Host validation of a decode call and its plan.  Returns the status; *empty
// is set when there is nothing to launch (num_seqs == 0, arguments valid).
static int decode_check(const void* q, int64_t q_row_stride, const void* k_cache,
                        const void* v_cache, int num_blocks, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* context_lens, void* out,
                        int64_t out_row_stride, int num_seqs, int max_context_len, int num_heads,
                        int num_kv_heads, int head_dim, int block_size, float scale, int dtype,
                        int cache_fp8, float k_scale, float v_scale, qw::DecodePlan* plan,
                        bool* empty) {
  *empty = false;
  if (cache_fp8) {
    const int st = check_fp8_scales(k_scale, v_scale);
    if (st) return st;
  }
  if (num_seqs < 0) return fail(QW_ERR_SHAPE, "num_seqs=%d < 0", num_seqs);
  if (num_seqs > 65535) return fail(QW_ERR_UNSUPPORTED, "num_seqs=%d > 65535", num_seqs);
  if (num_seqs == 0) {
    int st = check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype);
    *empty = st == QW_OK;
    return st;
  }
  int st = check_attn_common(q, q_row_stride, k_cache, v_cache, num_blocks, context_lens,
                             block_tables, max_blocks_per_seq, out, out_row_stride, num_seqs,
                             max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                             scale, dtype);
  if (st) return st;
  *plan = qw::plan_decode(num_seqs, max_context_len, num_heads, num_kv_heads, head_dim,
                          block_size, dtype, cache_fp8);
  return QW_OK;
}

static int decode_impl(const void* q, int64_t q_row_stride, const void* k_cache,
                       const void* v_cache, int num_blocks, const int32_t* block_tables,
                       int max_blocks_per_seq, const int32_t* context_lens, void* out,
                       int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                       int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, float scale, int dtype, int cache_fp8,
                       float k_scale, float v_scale, hipStream_t stream) {
  qw::DecodePlan plan{};
  bool empty = false;
  const int st = decode_check(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                              max_blocks_per_seq, context_lens, out, out_row_stride, num_seqs,
                              max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                              scale, dtype, cache_fp8, k_scale, v_scale, &plan, &empty);
  if (st) return st;
  if (empty) return ok();
  if (plan.ws_bytes > 0) {
    if (!workspace) return fail(QW_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", plan.ws_bytes);
    if (workspace_bytes < plan.ws_bytes)
      return fail(QW_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
    if (!aligned16(workspace)) return fail(QW_ERR_ALIGN, "workspace is not 16-byte aligned");
  }
  qw::AttnArgs a = decode_args(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, context_lens, out, out_row_stride, workspace,
                               workspace_bytes, num_seqs, max_context_len, num_heads,
                               num_kv_heads, head_dim, block_size, scale, dtype, cache_fp8,
                               k_scale, v_scale);
  const int est = current_error_word(&a.err);
  if (est) return est;
  return launched(qw::launch_decode(a, plan, stream));
}

int qwen2_attn_decode_paged(const void* q, int64_t q_row_stride, const void* k_cache,
                            const void* v_cache, int num_blocks, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* context_lens, void* out,
                            int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                            int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                            int head_dim, int block_size, float scale, int dtype,
                            hipStream_t stream) {
  return decode_impl(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, out, out_row_stride, workspace,
                     workspace_bytes, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim,
                     block_size, scale, dtype, 0, 1.0f, 1.0f, stream);
}

int qwen2_attn_decode_paged_fp8(const void* q, int64_t q_row_stride, const void* k_cache,
                                const void* v_cache, int num_blocks, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* context_lens, void* out,
                                int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                                int num_seqs, int max_context_len, int num_heads, int num_kv_heads,
                                int head_dim, int block_size, float scale, int dtype,
                                float k_scale, float v_scale, hipStream_t stream) {
  return decode_impl(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, out, out_row_stride, workspace,
                     workspace_bytes, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim,
                     block_size, scale, dtype, 1, k_scale, v_scale, stream);
}

}  // extern "C"

namespace {

// Decode workspace of qwen2_attn_decode_paged_noalloc: one static array per
// GPU (each device holds its own copy at its own address).  In host code the
// name `scratch` is only a stand-in for the symbol, never a device address:
// kernels get the address hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __align__(256) uint8_t scratch[QWEN2_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address (resolved on the first call there)
int current_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QW_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(QW_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QW_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return QW_OK;
}

}  // namespace

extern "C" {

int qwen2_attn_decode_paged_noalloc(const void* q, int64_t q_row_stride, const void* k_cache,
                                    const void* v_cache, int num_blocks,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, void* out,
                                    int64_t out_row_stride, int num_seqs, int max_context_len,
                                    int num_heads, int num_kv_heads, int head_dim, int block_size,
                                    float scale, int dtype, hipStream_t stream) {
  // validation, and the workspace this decode needs must fit the array:
  // both before the symbol lookup, so a refused call touches no device state
  qw::DecodePlan plan{};
  bool empty = false;
  const int vst = decode_check(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, context_lens, out, out_row_stride, num_seqs,
                               max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                               scale, dtype, 0, 1.0f, 1.0f, &plan, &empty);
  if (vst) return vst;
  if (empty) return ok();
  if (plan.ws_bytes > QWEN2_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(QW_ERR_WORKSPACE, "decode needs %zu bytes of workspace > the %zu-byte scratch",
                plan.ws_bytes, static_cast<size_t>(QWEN2_DECODE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  const int st = current_scratch(&ws);
  if (st) return st;
  return decode_impl(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, out, out_row_stride, ws,
                     QWEN2_DECODE_NOALLOC_SCRATCH_BYTES, num_seqs, max_context_len, num_heads,
                     num_kv_heads, head_dim, block_size, scale, dtype, 0, 1.0f, 1.0f, stream);
}

int qwen2_attn_decode_cascade_worthwhile(int num_prefixes, int num_prefix_members,
                                         int max_prefix_len, int num_kv_heads, int head_dim,
                                         int cache_fp8) {
  if (num_prefixes <= 0 || num_prefix_members <= num_prefixes || max_prefix_len <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0)
    return 0;
  const double saved = static_cast<double>(num_prefix_members - num_prefixes) * max_prefix_len *
                       num_kv_heads * 2.0 * head_dim * (cache_fp8 ? 1.0 : 2.0);
  return saved >= 96.0 * 1024.0 * 1024.0 ? 1 : 0;
}

size_t qwen2_attn_decode_cascade_workspace_size(int num_seqs, int max_context_len,
                                                int max_prefix_len, int num_prefixes,
                                                int num_prefix_members, int num_heads,
                                                int num_kv_heads, int head_dim, int block_size,
                                                int dtype) {
  if (num_seqs < 0 || max_context_len < 1 || max_prefix_len < 0 || num_prefixes < 0 ||
      num_prefix_members < 0)
    return static_cast<size_t>(-1);
  if (check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype)) return static_cast<size_t>(-1);
  return qw::plan_cascade(num_seqs, max_context_len, max_prefix_len, num_prefix_members,
                          num_prefixes, num_heads, num_kv_heads, head_dim, block_size, dtype, 0)
      .ws_bytes;
}

static int cascade_impl(const void* q, int64_t q_row_stride, const void* k_cache,
                        const void* v_cache, int num_blocks, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* prefix_indptr, const int32_t* prefix_seqs,
                        const int32_t* prefix_lens, int num_prefixes, int num_prefix_members,
                        int max_prefix_len, void* out, int64_t out_row_stride, void* workspace,
                        size_t workspace_bytes, int num_seqs, int max_context_len, int num_heads,
                        int num_kv_heads, int head_dim, int block_size, float scale, int dtype,
                        int cache_fp8, float k_scale, float v_scale, hipStream_t stream) {
  if (num_prefixes < 0 || num_prefix_members < 0 || max_prefix_len < 0)
    return fail(QW_ERR_SHAPE, "negative prefix-group size (num_prefixes=%d members=%d max_prefix_len=%d)",
                num_prefixes, num_prefix_members, max_prefix_len);
  if (num_prefixes > 0 && (!prefix_indptr || !prefix_lens))
    return fail(QW_ERR_NULL, "prefix_indptr/prefix_lens is NULL");
  if (num_prefix_members > 0 && !prefix_seqs) return fail(QW_ERR_NULL, "prefix_seqs is NULL");
  if (cache_fp8) {
    const int st = check_fp8_scales(k_scale, v_scale);
    if (st) return st;
  }
  if (num_seqs < 0) return fail(QW_ERR_SHAPE, "num_seqs=%d < 0", num_seqs);
  if (num_seqs > 65535) return fail(QW_ERR_UNSUPPORTED, "num_seqs=%d > 65535", num_seqs);
  if (num_seqs == 0) {
    int st = check_heads(num_heads, num_kv_heads, head_dim, block_size, dtype);
    return st ? st : ok();
  }
  int st = check_attn_common(q, q_row_stride, k_cache, v_cache, num_blocks, context_lens,
                             block_tables, max_blocks_per_seq, out, out_row_stride, num_seqs,
                             max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                             scale, dtype);
  if (st) return st;
  const qw::CascadePlan plan =
      qw::plan_cascade(num_seqs, max_context_len, max_prefix_len, num_prefix_members,
                       num_prefixes, num_heads, num_kv_heads, head_dim, block_size, dtype,
                       cache_fp8);
  if (plan.active && plan.tasks > 2147483646LL - 1)
    return fail(QW_ERR_SHAPE, "prefix level needs %lld workgroups", static_cast<long long>(plan.tasks));
  if (plan.ws_bytes > 0) {
    if (!workspace) return fail(QW_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", plan.ws_bytes);
    if (workspace_bytes < plan.ws_bytes)
      return fail(QW_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
    if (!aligned16(workspace)) return fail(QW_ERR_ALIGN, "workspace is not 16-byte aligned");
  }
  qw::AttnArgs a = decode_args(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, context_lens, out, out_row_stride, workspace,
                               workspace_bytes, num_seqs, max_context_len, num_heads,
                               num_kv_heads, head_dim, block_size, scale, dtype, cache_fp8,
                               k_scale, v_scale);
  const int est = current_error_word(&a.err);
  if (est) return est;
  qw::CascadeMeta m{};
  m.indptr = prefix_indptr;
  m.seqs = prefix_seqs;
  m.lens = prefix_lens;
  m.num_prefixes = num_prefixes;
  m.num_members = num_prefix_members;
  m.max_prefix_len = max_prefix_len;
  return launched(qw::launch_decode_cascade(a, m, plan, stream));
}

int qwen2_attn_decode_paged_cascade(const void* q, int64_t q_row_stride, const void* k_cache,
                                    const void* v_cache, int num_blocks,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, const int32_t* prefix_indptr,
                                    const int32_t* prefix_seqs, const int32_t* prefix_lens,
                                    int num_prefixes, int num_prefix_members, int max_prefix_len,
                                    void* out, int64_t out_row_stride, void* workspace,
                                    size_t workspace_bytes, int num_seqs, int max_context_len,
                                    int num_heads, int num_kv_heads, int head_dim, int block_size,
                                    float scale, int dtype, hipStream_t stream) {
  return cascade_impl(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                      max_blocks_per_seq, context_lens, prefix_indptr, prefix_seqs, prefix_lens,
                      num_prefixes, num_prefix_members, max_prefix_len, out, out_row_stride,
                      workspace, workspace_bytes, num_seqs, max_context_len, num_heads,
                      num_kv_heads, head_dim, block_size, scale, dtype, 0, 1.0f, 1.0f, stream);
}

int qwen2_attn_decode_paged_cascade_fp8(const void* q, int64_t q_row_stride, const void* k_cache,
                                        const void* v_cache, int num_blocks,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens,
                                        const int32_t* prefix_indptr, const int32_t* prefix_seqs,
                                        const int32_t* prefix_lens, int num_prefixes,
                                        int num_prefix_members, int max_prefix_len, void* out,
                                        int64_t out_row_stride, void* workspace,
                                        size_t workspace_bytes, int num_seqs,
                                        int max_context_len, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, float scale, int dtype,
                                        float k_scale, float v_scale, hipStream_t stream) {
  return cascade_impl(q, q_row_stride, k_cache, v_cache, num_blocks, block_tables,
                      max_blocks_per_seq, context_lens, prefix_indptr, prefix_seqs, prefix_lens,
                      num_prefixes, num_prefix_members, max_prefix_len, out, out_row_stride,
                      workspace, workspace_bytes, num_seqs, max_context_len, num_heads,
                      num_kv_heads, head_dim, block_size, scale, dtype, 1, k_scale, v_scale,
                      stream);
}

int qwen2_check_prefix_groups_host(const int32_t* prefix_indptr, const int32_t* prefix_seqs,
                                   const int32_t* prefix_lens, int num_prefixes,
                                   int num_prefix_members, int max_prefix_len,
                                   const int32_t* context_lens, const int32_t* block_tables,
                                   int num_seqs, int max_blocks_per_seq, int block_size) {
  if (num_prefixes < 0 || num_prefix_members < 0 || num_seqs < 0 || block_size < 1)
    return fail(QW_ERR_SHAPE, "negative sizes");
  if (num_prefixes == 0) return num_prefix_members == 0 ? ok()
                                : fail(QW_ERR_METADATA, "members without a group");
  if (!prefix_indptr || !prefix_lens || (num_prefix_members > 0 && !prefix_seqs) ||
      (num_seqs > 0 && (!context_lens || !block_tables)))
    return fail(QW_ERR_NULL, "NULL host array");
  if (prefix_indptr[0] != 0 || prefix_indptr[num_prefixes] != num_prefix_members)
    return fail(QW_ERR_METADATA, "prefix_indptr must run from 0 to %d", num_prefix_members);
  std::vector<char> seen(static_cast<size_t>(num_seqs), 0);
  for (int p = 0; p < num_prefixes; ++p) {
    const int i0 = prefix_indptr[p], i1 = prefix_indptr[p + 1];
    if (i1 < i0) return fail(QW_ERR_METADATA, "prefix_indptr decreases at group %d", p);
    const int L = prefix_lens[p];
    if (L <= 0 || L % block_size || L > max_prefix_len)
      return fail(QW_ERR_METADATA, "group %d: prefix length %d is not a positive multiple of %d up to %d",
                  p, L, block_size, max_prefix_len);
    const int nb = L / block_size;
    if (nb > max_blocks_per_seq)
      return fail(QW_ERR_METADATA, "group %d: prefix of %d blocks > max_blocks_per_seq", p, nb);
    for (int i = i0; i < i1; ++i) {
      const int s = prefix_seqs[i];
      if (s < 0 || s >= num_seqs)
        return fail(QW_ERR_METADATA, "group %d: member %d outside [0, %d)", p, s, num_seqs);
      if (seen[s]) return fail(QW_ERR_METADATA, "sequence %d is listed twice", s);
      seen[s] = 1;
      if (context_lens[s] <= L)
        return fail(QW_ERR_METADATA, "group %d: member %d has context %d <= prefix %d", p, s,
                    context_lens[s], L);
      const int32_t* bt = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
      const int32_t* b0 = block_tables + static_cast<int64_t>(prefix_seqs[i0]) * max_blocks_per_seq;
      for (int b = 0; b < nb; ++b)
        if (bt[b] != b0[b])
          return fail(QW_ERR_METADATA, "group %d: member %d names block %d at %d, the group %d", p,
                      s, bt[b], b, b0[b]);
    }
  }
  return ok();
}

int qwen2_check_metadata_host(const int32_t* positions, const int32_t* slot_mapping, int num_tokens,
                              const int32_t* cu_seqlens_q, const int32_t* context_lens,
                              const int32_t* block_tables, int num_seqs, int max_blocks_per_seq,
                              int num_blocks, int block_size, int max_position,
                              int max_context_len, int max_query_len) {
  if (num_tokens < 0 || num_seqs < 0) return fail(QW_ERR_SHAPE, "negative sizes");
  if (block_size < 1) return fail(QW_ERR_SHAPE, "block_size=%d < 1", block_size);
  if (num_seqs > 0 && (!context_lens || !block_tables))
    return fail(QW_ERR_NULL, "context_lens/block_tables is NULL");
  const int64_t nslots = static_cast<int64_t>(num_blocks) * block_size;
  if (positions) {
    for (int t = 0; t < num_tokens; ++t)
      if (positions[t] < 0 || positions[t] >= max_position)
        return fail(QW_ERR_METADATA, "positions[%d]=%d outside [0, %d)", t, positions[t], max_position);
  }
  if (slot_mapping) {
    std::vector<char> seen(static_cast<size_t>(nslots > 0 ? nslots : 0), 0);
    for (int t = 0; t < num_tokens; ++t) {
      const int sl = slot_mapping[t];
      if (sl == -1) continue;
      if (sl < -1 || sl >= nslots)
        return fail(QW_ERR_METADATA, "slot_mapping[%d]=%d outside [-1, %lld)", t, sl,
                    static_cast<long long>(nslots));
      if (seen[sl]) return fail(QW_ERR_METADATA, "slot %d named twice (token %d)", sl, t);
      seen[sl] = 1;
    }
  }
  if (cu_seqlens_q) {
    if (cu_seqlens_q[0] != 0) return fail(QW_ERR_METADATA, "cu_seqlens_q[0]=%d != 0", cu_seqlens_q[0]);
    if (cu_seqlens_q[num_seqs] > num_tokens)
      return fail(QW_ERR_METADATA, "cu_seqlens_q[%d]=%d > num_tokens=%d", num_seqs,
                  cu_seqlens_q[num_seqs], num_tokens);
  } else if (num_seqs > num_tokens && (positions || slot_mapping)) {
    return fail(QW_ERR_METADATA, "decode batch: num_seqs=%d > num_tokens=%d", num_seqs, num_tokens);
  }
  for (int s = 0; s < num_seqs; ++s) {
    const int r0 = cu_seqlens_q ? cu_seqlens_q[s] : s;
    const int n = cu_seqlens_q ? cu_seqlens_q[s + 1] - r0 : 1;
    const int c = context_lens[s];
    if (n < 0) return fail(QW_ERR_METADATA, "cu_seqlens_q decreases at sequence %d", s);
    if (n == 0) continue;
    if (c < n) return fail(QW_ERR_METADATA, "sequence %d: context %d < query rows %d", s, c, n);
    if (c > max_context_len)
      return fail(QW_ERR_METADATA, "sequence %d: context %d > max_context_len %d", s, c, max_context_len);
    if (max_query_len > 0 && n > max_query_len)
      return fail(QW_ERR_METADATA, "sequence %d: %d rows > max_query_len %d", s, n, max_query_len);
    const int nb = (c + block_size - 1) / block_size;
    if (nb > max_blocks_per_seq)
      return fail(QW_ERR_METADATA, "sequence %d needs %d blocks > max_blocks_per_seq %d", s, nb,
                  max_blocks_per_seq);
    const int32_t* bt = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
    for (int b = 0; b < nb; ++b)
      if (bt[b] < 0 || bt[b] >= num_blocks)
        return fail(QW_ERR_METADATA, "block_tables[%d][%d]=%d outside [0, %d)", s, b, bt[b], num_blocks);
    for (int i = 0; i < n; ++i) {
      const int t = r0 + i;
      const int p = c - n + i;
      if (positions && positions[t] != p)
        return fail(QW_ERR_METADATA, "positions[%d]=%d, expected %d (sequence %d row %d)", t,
                    positions[t], p, s, i);
      if (slot_mapping && slot_mapping[t] != -1) {
        const int64_t want = static_cast<int64_t>(bt[p / block_size]) * block_size + p % block_size;
        if (slot_mapping[t] != want)
          return fail(QW_ERR_METADATA, "slot_mapping[%d]=%d, block table gives %lld", t,
                      slot_mapping[t], static_cast<long long>(want));
      }
    }
  }
  return ok();
}

}  // extern "C"
