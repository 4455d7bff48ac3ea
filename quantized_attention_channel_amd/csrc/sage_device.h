// Device-side building blocks shared by the gfx950 kernels of libsage.
//
// Only gfx950 (CDNA4) is targeted: wave64, MFMA matrix cores with INT8 and
// OCP-FP8 operands, buffer loads with hardware range checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Method constants (quantisation blocks and the online-softmax KV tile).
constexpr int kBlkQ = 128;   // query tokens per INT8 scale
constexpr int kBlkK = 64;    // key tokens per INT8 scale
// Per-thread granularity: the tokens one lane holds in the attention kernel's
// matrix instructions (its single query; 16 consecutive keys of a 32-key block).
constexpr int kFineBlkQ = 1;
constexpr int kFineBlkK = 16;
constexpr int kBkv = 128;    // keys per online-softmax tile
constexpr int kVPad = 128;   // transposed-V rows are padded to a multiple of the tile
constexpr float kE4m3Max = 448.0f;
constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLog2E4m3Max = 8.807354922057604f;  // log2(448)

// ---------------------------------------------------------------- storage dtypes
// Inputs are 16-bit floats held as raw bits; conversions are exact (to fp32) or
// round-to-nearest-even (from fp32).
struct F16 {
  static __device__ __forceinline__ float to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  static __device__ __forceinline__ uint16_t from_f32(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};
struct BF16 {
  static __device__ __forceinline__ float to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
  static __device__ __forceinline__ uint16_t from_f32(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};

// ---------------------------------------------------------------- buffer loads
// A raw buffer resource over [base, base + bytes): loads at offsets outside it
// return zeros, which covers ragged sequence tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Bytes left in [0, bytes) from `start` on (0 past the end), as a wave-uniform
// (scalar) value. Every field of a buffer resource must be scalar: the
// compiler implements the saturating subtraction with a vector instruction,
// and a resource built from a vector value makes it wrap each load in a loop
// over the lanes' distinct resources.
__device__ __forceinline__ uint32_t tail_bytes(uint32_t bytes, uint32_t start) {
  return __builtin_amdgcn_readfirstlane(bytes > start ? bytes - start : 0u);
}
__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------- MFMA
// D(32x32) += A(32xK) B(Kx32). Lane l supplies row (l % 32) of A and column
// (l % 32) of B; lanes l and l+32 split the K range. The result lane l holds
// column (l % 32), rows 8*j + 4*(l / 32) + i in element 4*j + i.
__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = e4m3 for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_half(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_half(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- lane exchange
// Value of the same register in lane l ^ 32 combined with this lane's value.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a + b for two 16-bit floats, one packed dot instruction (products with 1.0 are exact).
__device__ __forceinline__ float dot2_ones(_Float16 a, _Float16 b, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(h2{a, b}, h2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
}
__device__ __forceinline__ float dot2_ones(__bf16 a, __bf16 b, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(b2{a, b}, b2{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}

}  // namespace sage
