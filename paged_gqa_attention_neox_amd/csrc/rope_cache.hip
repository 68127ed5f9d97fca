// Rotary table and the fused "rotate q/k + write k/v into the paged cache"
// kernel.  The rotation runs in float64 (the table too) and rounds once to
// the storage type, so the stored q/k equal the correctly rounded exact
// rotation; gfx950's float64 vector rate equals its float32 rate and the
// kernel is bound by HBM, not arithmetic.
//
// Rotary embedding over the whole head with base rope_theta
// ("Qwen2大模型架构解析与vLLM优化实践", §2.2 get_rope; "Qwen2 模型结构代码详解",
// §2 rope_theta = 1e6); NeoX pairing (i, i + d/2).  KV written into fixed-size
// blocks through a slot mapping ("vLLM 部署 Qwen", §2.1 PagedAttention).  The
// pages mention a fused RoPE kernel ("Qwen2大模型架构解析与vLLM优化实践", §7.3);
// here rotation and cache scatter are one pass over the fused QKV rows.
//
// The kernel is HBM-bound: per token it reads (H + 2 Hkv) * d elements and
// writes H * d (q_out) + 2 Hkv * d (cache) elements.  With an FP8 cache
// ("Qwen2大模型架构解析与vLLM优化实践", §4.1-4.2 FP8 KV-cache quantization with
// cache scales; §6.3 the E4M3FN format) the cache entries are E4M3FN codes of
// the exact rotated k (or v) divided by the tensor's scale, rounded once.  Each work item moves
// 16-byte vectors: 8 rotation pairs (x[i..i+8], x[i+d/2..]) of one head, or
// 8 elements of one v head.
#include "common.h"
#include "kernels.h"

namespace qw {

// ---------------------------------------------------------------------------
// cos/sin table in float64
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(double* __restrict__ tab, int max_position, int rot,
                                  double theta) {
  const int half = rot / 2;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(max_position) * half;
  if (idx >= total) return;
  const int p = static_cast<int>(idx / half);
  const int i = static_cast<int>(idx % half);
  const double f = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(rot));
  const double a = static_cast<double>(p) * f;
  double s, c;
  sincos(a, &s, &c);
  tab[static_cast<int64_t>(p) * rot + i] = c;
  tab[static_cast<int64_t>(p) * rot + half + i] = s;
}

hipError_t launch_rope_table(double* tab, int max_position, int rotary_dim, double theta,
                             hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(max_position) * (rotary_dim / 2);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                     stream, tab, max_position, rotary_dim, theta);
  return hipGetLastError();
}

// float64 -> bf16 with ONE rounding (round to nearest even).
// t = the float32 nearest to y.  Every bf16 value and every midpoint between
// two neighbouring bf16 values is a float32, and rounding is monotonic, so t
// never lies past a bf16 midpoint that y does not reach: rounding t to bf16
// gives the correctly rounded bf16 of y unless t sits exactly on a midpoint
// (its low 16 bits are 0x8000) that y is not on.  Then t is moved one float32
// step toward y, off the midpoint to y's side, and rounds the way y does.
// That case is rare (a float32 tie after an inexact first rounding), so it
// is handled under one branch for all N values, which a wave takes only when
// some lane needs it.
__device__ __forceinline__ float off_tie(float t, double y) {
  const uint32_t u = __float_as_uint(t);
  if ((u & 0xffffu) != 0x8000u || static_cast<double>(t) == y) return t;
  // |y| above |t|: one step away from zero (bit pattern + 1), else toward it
  return __uint_as_float(u + ((fabs(y) > fabs(static_cast<double>(t))) ? 1u : 0xffffffffu));
}
template <int N>
__device__ __forceinline__ void f64_to_bf16_pairs(const double (&y)[N], uint32_t (&w)[N / 2]) {
  float t[N];
  bool tie = false;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    t[j] = static_cast<float>(y[j]);
    tie |= (__float_as_uint(t[j]) & 0xffffu) == 0x8000u;
  }
  if (__builtin_expect(tie, 0)) {
#pragma unroll
    for (int j = 0; j < N; ++j) t[j] = off_tie(t[j], y[j]);
  }
#pragma unroll
  for (int j = 0; j < N / 2; ++j) w[j] = pack_bf16x2(t[2 * j], t[2 * j + 1]);
}

// float64 -> E4M3FN code with ONE rounding (nearest even), saturated at
// +-448: round to odd into fp32 (21 spare bits), clamp, then gfx950's
// v_cvt_pk_fp8_f32 (round to nearest even; it would turn magnitudes past the
// last rounding boundary into NaN, hence the clamp).
__device__ __forceinline__ float f64_to_f32_odd(double y) {
  const float t = __double2float_rz(y);
  uint32_t u = __float_as_uint(t);
  if (static_cast<double>(t) != y) u |= 1u;
  return fminf(fmaxf(__uint_as_float(u), -448.0f), 448.0f);
}
// eight codes from eight float64 values, as two little-endian words
__device__ __forceinline__ uint2 f64x8_to_fp8(const double (&y)[8]) {
  uint2 r;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(f64_to_f32_odd(y[0]), f64_to_f32_odd(y[1]), 0, false);
  r.x = __builtin_amdgcn_cvt_pk_fp8_f32(f64_to_f32_odd(y[2]), f64_to_f32_odd(y[3]), w, true);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(f64_to_f32_odd(y[4]), f64_to_f32_odd(y[5]), 0, false);
  r.y = __builtin_amdgcn_cvt_pk_fp8_f32(f64_to_f32_odd(y[6]), f64_to_f32_odd(y[7]), w, true);
  return r;
}

// ---------------------------------------------------------------------------
// 8-element vectors of the storage type
// ---------------------------------------------------------------------------
template <typename T> struct Vec8;

template <> struct Vec8<uint16_t> {   // bf16
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = w; }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
  __device__ __forceinline__ void from_f32(const float (&f)[8]) {
    w.x = pack_bf16x2(f[0], f[1]); w.y = pack_bf16x2(f[2], f[3]);
    w.z = pack_bf16x2(f[4], f[5]); w.w = pack_bf16x2(f[6], f[7]);
  }
  __device__ __forceinline__ uint16_t elem(int j) const {
    const uint32_t x = j < 2 ? w.x : j < 4 ? w.y : j < 6 ? w.z : w.w;
    return static_cast<uint16_t>((j & 1) ? (x >> 16) : (x & 0xffffu));
  }
  __device__ __forceinline__ void to_f64(double (&f)[8]) const {
    float t[8];
    to_f32(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = t[j];
  }
  __device__ __forceinline__ void from_f64(const double (&f)[8]) {
    uint32_t r[4];
    f64_to_bf16_pairs<8>(f, r);
    w = make_uint4(r[0], r[1], r[2], r[3]);
  }
  // two vectors rounded together (one rare-case branch for both)
  static __device__ __forceinline__ void from_f64_2(const double (&f1)[8], const double (&f2)[8],
                                                    Vec8& o1, Vec8& o2) {
    double f[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) { f[j] = f1[j]; f[8 + j] = f2[j]; }
    uint32_t r[8];
    f64_to_bf16_pairs<16>(f, r);
    o1.w = make_uint4(r[0], r[1], r[2], r[3]);
    o2.w = make_uint4(r[4], r[5], r[6], r[7]);
  }
  static __device__ __forceinline__ uint16_t nan() { return 0x7fc0; }
};

template <> struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<float4*>(p) = a;
    *reinterpret_cast<float4*>(p + 4) = b;
  }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ void from_f32(const float (&f)[8]) {
    a = make_float4(f[0], f[1], f[2], f[3]);
    b = make_float4(f[4], f[5], f[6], f[7]);
  }
  __device__ __forceinline__ float elem(int j) const {
    return j == 0 ? a.x : j == 1 ? a.y : j == 2 ? a.z : j == 3 ? a.w
         : j == 4 ? b.x : j == 5 ? b.y : j == 6 ? b.z : b.w;
  }
  __device__ __forceinline__ void to_f64(double (&f)[8]) const {
    float t[8];
    to_f32(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = t[j];
  }
  __device__ __forceinline__ void from_f64(const double (&f)[8]) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = static_cast<float>(f[j]);   // one rounding, nearest even
    from_f32(t);
  }
  static __device__ __forceinline__ void from_f64_2(const double (&f1)[8], const double (&f2)[8],
                                                    Vec8& o1, Vec8& o2) {
    o1.from_f64(f1);
    o2.from_f64(f2);
  }
  static __device__ __forceinline__ float nan() { return __builtin_nanf(""); }
};

// ---------------------------------------------------------------------------
// fused rotate + scatter
// ---------------------------------------------------------------------------
// A rotation item is one 8-pair chunk (pairs i0 .. i0 + 7) of RH heads of
// one token: the chunk's cos/sin (128 bytes of the table row) is read once
// for the RH heads, and the RH heads' input loads are in flight together.
// RH = 2 for batches of at least 512 tokens (more bytes in flight per wave;
// measured on the 2463-token prefill batch: 13.9 us with one head per item,
// 12.0 with two, 12.1 with four); RH = 1 for smaller batches (more items to
// spread: 64 tokens 3.8 against 4.0 us) and for FP8 caches, whose encoding
// needs the registers (17.0 against 18.2 us).  With the q/k norm the
// prefill batch takes 16.0 us with two heads, 16.4 with one.

// CF8: the caches hold E4M3FN codes of (rotated) k / k_scale and v / v_scale.
// QKN: Qwen3 q/k norm before the rotation ("nano-vllm: Qwen3 骨架", §5 the
// q_norm / k_norm RMSNorm modules of the attention; §3.2 rms_norm_eps): each
// q and k head becomes x / sqrt(mean(x^2) + eps) * w in float64.  The RCH
// chunk items of a head group sit in RCH consecutive lanes aligned to RCH
// (per-token item counts are multiples of RCH), so a head's sum of squares
// needs log2(RCH) lane exchanges.
template <typename T, int D, bool CF8, bool QKN, int kRH>
__global__ __launch_bounds__(256) void rope_cache_write_kernel(RopeWriteArgs a) {
  constexpr int HALF = D / 2;
  constexpr int RCH = HALF / 8;   // chunks of 8 pairs per head
  constexpr int VCH = D / 8;      // v items per head (8 elements each)
  const int B = a.block_size;     // tokens per cache block: 16, 32 or 64 (validated on the host)
  const int lb = 31 - __builtin_clz(B);
  const int H = a.num_heads, Hkv = a.num_kv_heads;
  const int NH = H + Hkv;                         // rotated heads per token
  const int rot_items = (NH + kRH - 1) / kRH * RCH;
  const int vch = Hkv * VCH;                      // v items per token
  // Item space: the rotation items token by token, then (from a wave
  // boundary) the v items in groups of 16 tokens with the token fastest, so
  // that the 16 lanes storing one dims row of a V tile ([d][B]) hold 16
  // consecutive tokens: with consecutive slots (a prefill's block) their
  // 2-byte stores fill whole 32-byte rows instead of touching one row each.
  const int64_t rot_total = static_cast<int64_t>(a.num_tokens) * rot_items;
  const int64_t v_base = (rot_total + 63) / 64 * 64;
  const int64_t total = v_base + (static_cast<int64_t>(a.num_tokens) + 15) / 16 * 16 * vch;
  const int64_t cache_slots = static_cast<int64_t>(a.num_blocks) * B;

  const T* q = static_cast<const T*>(a.q);            // may alias q_out (in place)
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  T* q_out = static_cast<T*>(a.q_out);
  T* __restrict__ kc = static_cast<T*>(a.k_cache);
  T* __restrict__ vc = static_cast<T*>(a.v_cache);
  uint8_t* __restrict__ kc8 = static_cast<uint8_t*>(a.k_cache);
  uint8_t* __restrict__ vc8 = static_cast<uint8_t*>(a.v_cache);
  const double ks = a.k_scale, vs = a.v_scale;

  // 32-bit item arithmetic when the items fit (the usual case)
  const bool narrow = total <= 0x7fffffff;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (idx < rot_total) {
      // ---- rotation item: chunk i0 of heads hg * kRH .. hg * kRH + kRH - 1 ----
      const int t = narrow ? static_cast<int>(static_cast<uint32_t>(idx) / static_cast<uint32_t>(rot_items))
                           : static_cast<int>(idx / rot_items);
      const int w = static_cast<int>(idx - static_cast<int64_t>(t) * rot_items);
      const int hg = w / RCH;
      const int i0 = (w - hg * RCH) * 8;
      // the input vectors are loaded first: their addresses do not depend on
      // the position or slot, so these loads and the metadata loads are in
      // flight together
      Vec8<T> x1v[kRH], x2v[kRH];
#pragma unroll
      for (int r = 0; r < kRH; ++r) {
        const int head = hg * kRH + r;
        if (head < NH) {
          const T* src = head < H ? q + static_cast<int64_t>(t) * a.q_stride + static_cast<int64_t>(head) * D
                                  : k + static_cast<int64_t>(t) * a.k_stride + static_cast<int64_t>(head - H) * D;
          x1v[r].load(src + i0);
          x2v[r].load(src + HALF + i0);
        }
      }
      const int pos = a.positions[t];
      const int slot = a.slots[t];
      const bool pos_ok = static_cast<unsigned>(pos) < static_cast<unsigned>(a.max_position);
      const bool slot_ok = slot >= 0 && static_cast<int64_t>(slot) < cache_slots;
      if (!pos_ok) report_error(a.err, kErrPosition);
      if (!slot_ok && slot != -1) report_error(a.err, kErrSlot);
      const int64_t blk = slot_ok ? slot >> lb : 0;
      const int off = slot_ok ? slot & (B - 1) : 0;
      double cv[8], sv[8];
      if (pos_ok) {
        const double* cs = a.cos_sin + static_cast<int64_t>(pos) * D;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const double2 c2 = *reinterpret_cast<const double2*>(cs + i0 + j);
          const double2 s2 = *reinterpret_cast<const double2*>(cs + HALF + i0 + j);
          cv[j] = c2.x; cv[j + 1] = c2.y;
          sv[j] = s2.x; sv[j + 1] = s2.y;
        }
      }
#pragma unroll
      for (int r = 0; r < kRH; ++r) {
        const int head = hg * kRH + r;            // uniform across the RCH lanes of a head group
        if (head >= NH) break;
        const bool is_q = head < H;
        if (!is_q && !(pos_ok && slot_ok)) continue;
        T* dst;
        if (is_q) {
          dst = q_out + static_cast<int64_t>(t) * a.q_out_stride + static_cast<int64_t>(head) * D;
          if (!pos_ok) {
            Vec8<T> nanv;
            float f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = __builtin_nanf("");
            nanv.from_f32(f);
            nanv.store(dst + i0);
            nanv.store(dst + HALF + i0);
            continue;
          }
        } else {
          const int gk = head - H;
          dst = CF8 ? nullptr : kc + ((blk * Hkv + gk) * B + off) * D;
        }
        double x1[8], x2[8], y1[8], y2[8];
        x1v[r].to_f64(x1);
        x2v[r].to_f64(x2);
        if constexpr (QKN) {
          double ss = 0.0;
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fma(x1[j], x1[j], fma(x2[j], x2[j], ss));
#pragma unroll
          for (int o = 1; o < RCH; o <<= 1) ss += __shfl_xor(ss, o);
          // x / rms as x * (1 / rms): one float64 division per head instead
          // of one per element (the product differs from the quotient by at
          // most an ulp or two of float64, far below the single rounding to
          // the storage type)
          const double inv_rms = 1.0 / sqrt(ss / D + a.rms_eps);
          const T* wp = static_cast<const T*>(is_q ? a.q_norm_w : a.k_norm_w);
          Vec8<T> w1v, w2v;
          w1v.load(wp + i0);
          w2v.load(wp + HALF + i0);
          double w1[8], w2[8];
          w1v.to_f64(w1);
          w2v.to_f64(w2);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x1[j] = x1[j] * inv_rms * w1[j];
            x2[j] = x2[j] * inv_rms * w2[j];
          }
        }
        // float64 rotation: the inputs are exact, each output is rounded once
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          y1[j] = fma(x1[j], cv[j], -(x2[j] * sv[j]));
          y2[j] = fma(x2[j], cv[j], x1[j] * sv[j]);
        }
        if (CF8 && !is_q) {
          // the code of the rotation divided by the scale: a correctly
          // rounded float64 quotient, then one rounding to the code
          double z1[8], z2[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            z1[j] = y1[j] / ks;
            z2[j] = y2[j] / ks;
          }
          uint8_t* d8 = kc8 + ((blk * Hkv + (head - H)) * B + off) * D;
          *reinterpret_cast<uint2*>(d8 + i0) = f64x8_to_fp8(z1);
          *reinterpret_cast<uint2*>(d8 + HALF + i0) = f64x8_to_fp8(z2);
          continue;
        }
        Vec8<T> o1, o2;
        Vec8<T>::from_f64_2(y1, y2, o1, o2);
        o1.store(dst + i0);
        o2.store(dst + HALF + i0);
      }
    } else {
      // ---- v item: 8 elements of one v head of one token ----
      if (idx < v_base) continue;
      const int64_t vi = idx - v_base;
      const int64_t rest = vi >> 4;
      const int64_t th = narrow ? static_cast<int64_t>(static_cast<uint32_t>(rest) / static_cast<uint32_t>(vch))
                                : rest / vch;
      const int t = static_cast<int>(th * 16 + (vi & 15));
      const int wv = static_cast<int>(rest - th * vch);
      if (t >= a.num_tokens) continue;
      const int gv = wv / VCH;
      const int e0 = (wv - gv * VCH) * 8;
      Vec8<T> x;
      x.load(v + static_cast<int64_t>(t) * a.v_stride + static_cast<int64_t>(gv) * D + e0);
      const int pos = a.positions[t];
      const int slot = a.slots[t];
      const bool pos_ok = static_cast<unsigned>(pos) < static_cast<unsigned>(a.max_position);
      const bool slot_ok = slot >= 0 && static_cast<int64_t>(slot) < cache_slots;
      if (!(pos_ok && slot_ok)) continue;
      const int64_t blk = slot >> lb;
      const int off = slot & (B - 1);
      if (CF8) {
        double xv[8];
        x.to_f64(xv);
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] /= vs;
        const uint2 c8 = f64x8_to_fp8(xv);
        uint8_t* d8 = vc8 + ((blk * Hkv + gv) * D + e0) * B + off;   // V tile is [d][B]
#pragma unroll
        for (int j = 0; j < 8; ++j) d8[j * B] = static_cast<uint8_t>(((j < 4 ? c8.x : c8.y) >> (8 * (j & 3))) & 0xff);
        continue;
      }
      T* dst = vc + ((blk * Hkv + gv) * D + e0) * B + off;     // V tile is [d][B]
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j * B] = x.elem(j);
    }
  }
}

hipError_t launch_rope_cache_write(const RopeWriteArgs& a, hipStream_t stream) {
  const int d = a.head_dim;
  // the kernel's item space: rotation items, then v items padded to whole
  // waves and groups of 16 tokens
  const int RH = a.cache_fp8 || a.num_tokens < 512 ? 1 : 2;   // heads per rotation item
  const int64_t rot_total = static_cast<int64_t>(a.num_tokens) *
                            ((a.num_heads + a.num_kv_heads + RH - 1) / RH) * (d / 16);
  const int64_t total = (rot_total + 63) / 64 * 64 +
                        (static_cast<int64_t>(a.num_tokens) + 15) / 16 * 16 * a.num_kv_heads * (d / 8);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 1 << 20) blocks = 1 << 20;
  const dim3 grid(static_cast<unsigned>(blocks)), block(threads);
#define QW_ROPE_LAUNCH(T, D, F8, N)                                                          \
  do {                                                                                       \
    if (RH == 2)                                                                             \
      hipLaunchKernelGGL((rope_cache_write_kernel<T, D, F8, N, 2>), grid, block, 0, stream, a); \
    else                                                                                     \
      hipLaunchKernelGGL((rope_cache_write_kernel<T, D, F8, N, 1>), grid, block, 0, stream, a); \
  } while (0)
#define QW_ROPE_D(T, F8, N) \
  do { if (d == 128) QW_ROPE_LAUNCH(T, 128, F8, N); else QW_ROPE_LAUNCH(T, 64, F8, N); } while (0)
#define QW_ROPE_N(T, F8) \
  do { if (a.q_norm_w) QW_ROPE_D(T, F8, true); else QW_ROPE_D(T, F8, false); } while (0)
  if (a.dtype == kBF16) {
    if (a.cache_fp8) QW_ROPE_N(uint16_t, true); else QW_ROPE_N(uint16_t, false);
  } else {
    if (a.cache_fp8) QW_ROPE_N(float, true); else QW_ROPE_N(float, false);
  }
#undef QW_ROPE_N
#undef QW_ROPE_D
#undef QW_ROPE_LAUNCH
  return hipGetLastError();
}

}  // namespace qw
