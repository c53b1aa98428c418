// bf16 -> MXFP4 quantization kernels for gfx950.
//
// Format (block-scaled E2M1 operands of the EFQ-Softmax abstract; microscaling
// FP4 of the SageAttention3 title): 32 consecutive elements of the contraction
// axis share one E8M0 scale 2^e, e = clamp(floor(log2 amax) - 2, -127, 127);
// each element becomes round-to-nearest-even(x / 2^e) on the E2M1 grid,
// saturating at 6, sign kept.  The hardware conversion v_cvt_scalef32_pk_fp4_f32
// implements exactly that element rule (divide by the scale, RNE with ties to
// the even code, saturation, signed zero); it is fed x * 2^-e, which is exact,
// with a unit scale, so that the e = -127 case never needs a subnormal scale.
//
// Both kernels are streaming and HBM-bound: 2 bytes read and 0.5 + 1/32 bytes
// written per element.
#include "common.h"
#include "internal.h"

namespace attnfp4 {

// ---- axis 0 (Q, K): blocks along the contiguous last axis -------------------------------
// One lane converts 8 consecutive elements (one 16-byte load); the four lanes of a DPP quad
// form one 32-element block and agree on its scale through two quad permutations.  A thread
// takes RQ_PER such groups, 256 groups apart, with all its loads issued before the first
// conversion; the loads are non-temporal (the input is read once).  Measured on one bench-shape
// tensor (24 x 32768 x 128): 41 us against 46 us for one group per thread in a grid-stride loop.
constexpr int RQ_PER = 4;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) quantize_rows_kernel(const uint4* __restrict__ x,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t n8) {
  const int64_t base = (int64_t)blockIdx.x * (256 * RQ_PER) + threadIdx.x;
  v4u w[RQ_PER];
#pragma unroll
  for (int p = 0; p < RQ_PER; ++p) {
    const int64_t g = base + 256 * p;
    w[p] = g < n8 ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + g)) : v4u{0, 0, 0, 0};
  }
#pragma unroll
  for (int p = 0; p < RQ_PER; ++p) {
    const int64_t g = base + 256 * p;     // quads stay whole: n8 is a multiple of 4
    if (g >= n8) return;
    float f[8] = {bf16_lo(w[p][0]), bf16_hi(w[p][0]), bf16_lo(w[p][1]), bf16_hi(w[p][1]),
                  bf16_lo(w[p][2]), bf16_hi(w[p][2]), bf16_lo(w[p][3]), bf16_hi(w[p][3])};
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, __float_as_uint(f[i]) & 0x7FFFFFFFu);
    // quad max: xor 1 then xor 2 (quad_perm [1,0,3,2] and [2,3,0,1])
    amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
    amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, false));
    const int sbyte = mx_scale_byte_from_amax_bits(amax);
    const float inv = exp2i(127 - sbyte);                    // 2^-e, e = sbyte - 127
    uint32_t c = 0;
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[0] * inv, f[1] * inv, 1.0f, 0);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[2] * inv, f[3] * inv, 1.0f, 1);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[4] * inv, f[5] * inv, 1.0f, 2);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[6] * inv, f[7] * inv, 1.0f, 3);
    codes[g] = c;
    if ((g & 3) == 0) scales[g >> 2] = (uint8_t)sbyte;
  }
}

// ---- axis 1 (V): blocks along the sequence, written block-major --------------------------
// Output layout [n/32][d][16 code bytes] and [n/32][d] scales: the codes of one 32-token block
// for every channel, then the next block, so that a 64-key tile of V^ is one contiguous run.
// One thread per (32-token block, channel pair): it reads the pair's 32 tokens straight from
// global memory (consecutive threads hold consecutive channel pairs, so each of the 32 loads of
// a wave is one contiguous 256-byte row segment), converts its two MX blocks and writes their
// 2 x 16 code bytes and two scale bytes next to those of the neighbouring pairs.  No LDS and no
// barrier: every wave keeps its 32 (non-temporal) loads in flight.  Measured on one bench-shape
// tensor: 40 us, against 45-56 us for the earlier LDS-staged form.
__global__ void __launch_bounds__(256) quantize_cols_kernel(const uint32_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t n, int64_t d, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t dp = d / 2, nb = n / 32;
  const int64_t cp = idx % dp, rest = idx / dp;   // channel pair; (head, block)
  const int64_t blk = rest % nb, bh = rest / nb;
  const uint32_t* xs = x + (bh * n + blk * 32) * dp + cp;
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = __builtin_nontemporal_load(xs + (int64_t)i * dp);
  uint32_t a0 = 0, a1 = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    a0 = max(a0, (w[i] << 16) & 0x7FFFFFFFu);
    a1 = max(a1, w[i] & 0x7FFF0000u);
  }
  const int s0 = mx_scale_byte_from_amax_bits(a0), s1 = mx_scale_byte_from_amax_bits(a1);
  const float i0 = exp2i(127 - s0), i1 = exp2i(127 - s1);
  uint32_t c0w[4], c1w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t* v = w + 8 * q;
    uint32_t u = 0, t = 0;
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, bf16_lo(v[0]) * i0, bf16_lo(v[1]) * i0, 1.0f, 0);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, bf16_lo(v[2]) * i0, bf16_lo(v[3]) * i0, 1.0f, 1);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, bf16_lo(v[4]) * i0, bf16_lo(v[5]) * i0, 1.0f, 2);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, bf16_lo(v[6]) * i0, bf16_lo(v[7]) * i0, 1.0f, 3);
    t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, bf16_hi(v[0]) * i1, bf16_hi(v[1]) * i1, 1.0f, 0);
    t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, bf16_hi(v[2]) * i1, bf16_hi(v[3]) * i1, 1.0f, 1);
    t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, bf16_hi(v[4]) * i1, bf16_hi(v[5]) * i1, 1.0f, 2);
    t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, bf16_hi(v[6]) * i1, bf16_hi(v[7]) * i1, 1.0f, 3);
    c0w[q] = u;
    c1w[q] = t;
  }
  const int64_t ch0 = 2 * cp;
  uint8_t* cb = codes + bh * d * (n / 2) + (blk * d + ch0) * 16;
  *reinterpret_cast<uint4*>(cb) = make_uint4(c0w[0], c0w[1], c0w[2], c0w[3]);
  *reinterpret_cast<uint4*>(cb + 16) = make_uint4(c1w[0], c1w[1], c1w[2], c1w[3]);
  *reinterpret_cast<uint16_t*>(scales + bh * d * (n / 32) + blk * d + ch0) = (uint16_t)(s0 | (s1 << 8));
}

hipError_t launch_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int axis, void* codes,
                           void* scales, hipStream_t stream) {
  if (axis == 0) {
    const int64_t n8 = bh * n * d / 8;
    const int64_t blocks = (n8 + 256 * RQ_PER - 1) / (256 * RQ_PER);
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)x, (uint32_t*)codes, (uint8_t*)scales, n8);
  } else {
    const int64_t total = bh * (n / 32) * (d / 2);   // (block, channel pair) items
    hipLaunchKernelGGL(quantize_cols_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       (const uint32_t*)x, (uint8_t*)codes, (uint8_t*)scales, n, d, total);
  }
  return hipGetLastError();
}

}  // namespace attnfp4
