// Device helpers shared by the gfx950 kernels: bf16 <-> fp32, wave-level
// DPP reductions, vector loads.  CDNA4 wavefronts are 64 lanes wide.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qw {

constexpr int kWave = 64;

// ---- bf16 storage (raw 16-bit patterns) ------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// low / high bf16 of a packed pair, widened exactly
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even, with gfx950's v_cvt_pk_bf16_f32 (a
// NaN stays a NaN).  The two-element vector conversion selects it; a scalar
// conversion would be expanded into integer rounding code.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
}

// ---- DPP lane exchange (within rows of 16 lanes) ---------------------------
// dpp_ctrl encodings (GFX9 family): quad_perm [a,b,c,d] = a|b<<2|c<<4|d<<6,
// row_ror:n = 0x120+n, row_mirror = 0x140, row_half_mirror = 0x141.
// Every control used here reads a valid lane, so bound_ctrl does not change
// the result; with it set the compiler fuses "mov_dpp + add" into one
// v_add_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16

// Sum over aligned groups of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---- bf16 dot product of packed pairs, fp32 accumulate (v_dot2_f32_bf16) --
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
// First product of a chain: the three-operand form with an inline zero
// accumulator (the two-operand accumulate-in-place form would need a zeroing
// move first).
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Device error word: kernels that meet metadata outside its contract (a
// position, slot, block id or sequence length out of range) OR one of these
// flags into the word (err may be null: no report).  Only the error path
// touches it.  The values are those of QW_DEVICE_ERR_* in the public header.
constexpr unsigned kErrPosition = 1u, kErrSlot = 2u, kErrBlock = 4u, kErrSequence = 8u;
__device__ __forceinline__ void report_error(unsigned* err, unsigned flag) {
  if (err) atomicOr(err, flag);
}

}  // namespace qw
