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
// form one 32-element block and agree on its scale through two quad permutations.
__global__ void __launch_bounds__(256) quantize_rows_kernel(const uint4* __restrict__ x,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;   // multiple of 4: quads stay whole
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n8; g += stride) {
    uint4 w = x[g];
    float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                  bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
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
// Grid (ceil(n / 128), ceil(d / 128), bh); 256 threads per 128-token x 128-channel tile.  The tile
// is read with coalesced 16-byte loads into LDS ([token][channel pair], 272-byte rows), then each
// thread takes one channel pair and one 32-token block: two complete MX blocks, whose 16 code
// bytes per channel land next to those of the neighbouring channels.
constexpr int QC_TOK = 128, QC_CH = 128, QC_PITCH = 68;   // dwords per LDS row (64 + 4 padding)
__global__ void __launch_bounds__(256) quantize_cols_kernel(const uint32_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t n, int64_t d) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[QC_TOK * QC_PITCH];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * QC_TOK, c0 = (int64_t)blockIdx.y * QC_CH;
  const int ntok = (int)min((int64_t)QC_TOK, n - t0);       // multiple of 32
  const int nch = (int)min((int64_t)QC_CH, d - c0);         // multiple of 32
  const uint32_t* xs = x + (bh * n + t0) * (d / 2) + c0 / 2;
  for (int k = tid; k < QC_TOK * 16; k += 256) {
    const int r = k >> 4, cc = k & 15;                      // token, 8-channel chunk
    if (r < ntok && 8 * cc < nch)
      *reinterpret_cast<uint4*>(&tile[r * QC_PITCH + 4 * cc]) =
          *reinterpret_cast<const uint4*>(xs + (int64_t)r * (d / 2) + 4 * cc);
  }
  __syncthreads();
  const int cp = tid & 63, tb = tid >> 6;                   // channel pair, 32-token block
  if (2 * cp >= nch || 32 * tb >= ntok) return;
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = tile[(32 * tb + i) * QC_PITCH + cp];
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
  const int64_t ch0 = c0 + 2 * cp;
  const int64_t blk = (t0 >> 5) + tb;               // 32-token block
  uint8_t* cb = codes + bh * d * (n / 2) + (blk * d + ch0) * 16;
  *reinterpret_cast<uint4*>(cb) = make_uint4(c0w[0], c0w[1], c0w[2], c0w[3]);
  *reinterpret_cast<uint4*>(cb + 16) = make_uint4(c1w[0], c1w[1], c1w[2], c1w[3]);
  *reinterpret_cast<uint16_t*>(scales + bh * d * (n / 32) + blk * d + ch0) = (uint16_t)(s0 | (s1 << 8));
}

hipError_t launch_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int axis, void* codes,
                           void* scales, hipStream_t stream) {
  if (axis == 0) {
    const int64_t n8 = bh * n * d / 8;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)x, (uint32_t*)codes, (uint8_t*)scales, n8);
  } else {
    dim3 grid((unsigned)((n + QC_TOK - 1) / QC_TOK), (unsigned)((d + QC_CH - 1) / QC_CH), (unsigned)bh);
    hipLaunchKernelGGL(quantize_cols_kernel, grid, dim3(256), 0, stream, (const uint32_t*)x,
                       (uint8_t*)codes, (uint8_t*)scales, n, d);
  }
  return hipGetLastError();
}

}  // namespace attnfp4
