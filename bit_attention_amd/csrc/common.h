// Internal helpers shared by the gfx950 kernels of libattnfp4 (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attnfp4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Key held by row r (0..31) of a 32x32 S^T MFMA tile: r = 8a + 4b + c -> key 16b + 4a + c.  With
// the 32x32 MFMA output layout (register i of lane l is row 8(i/4) + 4(l/32) + i%4) this puts key
// 16(l/32) + i in register i of lane l, i.e. each lane holds 16 consecutive keys.
__device__ __forceinline__ int row_key(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// XOR swizzles of 16-byte chunks in LDS rows, chosen so that the MFMA operand reads (consecutive
// lanes reading consecutive rows at one logical chunk, 16-byte per lane) hit distinct 16-byte bank
// groups whether the LDS serves 8 or 16 such lanes per cycle.
//  - rows of 64 B (4 chunks) or 32 B (2 chunks), as for the FP4 operand tiles:
__device__ __forceinline__ int swz_small(int row, int nchunks) { return ((row >> 1) ^ (row >> 2)) & (nchunks - 1); }
//  - rows of 256 B (16 chunks) or 128 B (8 chunks), as for the bf16 operand tiles:
__device__ __forceinline__ int swz_big(int row, int nchunks) {
  return nchunks == 16 ? (row & 15) : ((row ^ (row >> 3)) & 7);
}

// Raw buffer resource over [base, base + bytes) (gfx9 dword 3; out-of-range loads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  v2bf v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// E8M0 exponent of the MX block scale from the block's max magnitude (fp32 bits):
// e = clamp(floor(log2 amax) - 2, -127, 127), with amax < 2^-126 counted as 2^-127.
// For a finite fp32 amax the biased exponent field E gives floor(log2 amax) = E - 127
// (E = 0 for zero and subnormals, which yields the -127 of the rule), so the scale
// byte e + 127 is max(E - 2, 0).
__device__ __forceinline__ int mx_scale_byte_from_amax_bits(uint32_t amax_bits) {
  int field = (int)((amax_bits >> 23) & 0xFF);
  return field > 2 ? field - 2 : 0;
}

// 2^k as an fp32 for k in [-126, 127].
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

}  // namespace attnfp4
