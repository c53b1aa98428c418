// NVFP4-style operands on gfx950: E2M1 codes in 16-element blocks with an FP8 E4M3 block scale
// and one fp32 scale per tensor, and the attention forward over them.
//
// The pages name NVFP4 (TetraJet-v2 abstract) and compare it with MXFP4 and HiF4 (RFQ and HiFA4
// abstracts) without defining it.  The format implemented here is the published NVFP4 layout, with
// every rounding step taken in fp32 with round-to-nearest-even:
//   G = max(amax_tensor / 2688, 2^-117)          2688 = 6 * 448 (E2M1 max times E4M3 max)
//   per block of 16: s = amax_block / (6 G), S = E4M3(s) (ties to even, saturating at 448),
//   sigma = S G, code = E2M1(x / sigma) (ties to even, saturating at 6, sign kept; sign only
//   when S = 0); value = G * S * E2M1(code).
//
// gfx950's block-scaled matrix core takes power-of-two scales per 32 elements only, so this format
// runs on the fp16 matrix core: the product of an E2M1 value (at most 2 significant bits) and an
// E4M3 scale (at most 4) has at most 6 significant bits and lies in [2^-10, 2688], so E2M1 * S is
// exact in fp16 (normal range 2^-14 .. 65504), every fp16 product is exact in the fp32
// accumulator, and the tensor scales are applied once to the fp32 scores and outputs.  fp16
// rather than bf16 because its packed multiply and dot instructions let the probabilities be
// rebuilt two at a time.
//
// The probabilities are requantized in the same format per 16 keys (the tensor scale of P is the
// one for amax = 1, as p <= 1 with equality at the row maximum): S = E4M3(max p * 448), P~ =
// E2M1(p * 2688 / S) * S / 2688; the factor 1/2688 cancels between the numerator and the
// denominator and is applied to the saved row sum only.
#include "common.h"
#include "internal.h"

namespace attnfp4 {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNvDiv = 2688.0f;
constexpr float kLog2NvDiv = 11.392317422778760f;    // log2(2688)
constexpr float kNvGMin = 6.018531076210112e-36f;   // 2^-117

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v16f mfma_f16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// Two fp32 values that are exact in fp16 -> packed fp16.
__device__ __forceinline__ uint32_t pk_f16_exact(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Nearest E4M3 value to t >= 0 (finite), ties to the even mantissa, saturating at 448.  The
// quantum of t's binade is 2^(floor(log2 t) - 3), and 2^-9 below 2^-6 (subnormals); scaling by a
// power of two is exact and v_rndne_f32 rounds half to even.
__device__ __forceinline__ float e4m3_round(float t) {
  const int e = (int)(__float_as_uint(t) >> 23) - 127;       // floor(log2 t); -127 for 0, subnormals
  const int qe = max(e, -6) - 3;
  return fminf(__builtin_rintf(t * exp2i(-qe)) * exp2i(qe), 448.0f);
}

// E4M3 byte of a value produced by e4m3_round.
__device__ __forceinline__ uint32_t e4m3_byte(float r) {
  if (r < 0.015625f) return (uint32_t)(r * 512.0f);          // subnormal: r = m 2^-9
  const uint32_t u = __float_as_uint(r);
  return ((((u >> 23) & 0xFF) - 120) << 3) | ((u >> 20) & 7);  // exponent field - 127 + 7
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15, m = b & 7;
  return e == 0 ? (float)m * 0.001953125f : (float)(8 + m) * exp2i((int)e - 10);
}

// Tensor scale from the tensor's amax (fp32 bits).
__device__ __forceinline__ float nv_tensor_scale(uint32_t amax_bits) {
  return fmaxf(__uint_as_float(amax_bits) / kNvDiv, kNvGMin);
}

// 8 codes (one dword) of 8 values already divided by the block's sigma.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* v) {
  uint32_t c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[0], v[1], 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[2], v[3], 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[4], v[5], 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[6], v[7], 1.0f, 3);
  return c;
}

// ---- tensor amax ------------------------------------------------------------------------------
__global__ void nv_amax_clear_kernel(float* ts) { reinterpret_cast<uint32_t*>(ts)[1] = 0u; }

// Largest |x| over the tensor into ts[1] (fp32 bits; non-negative floats order as unsigned ints).
// Four 16-byte loads in flight per lane; one atomic per workgroup.
__device__ __forceinline__ uint32_t bf16x8_absmax(uint4 w) {
  const uint32_t m0 = max(max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu), max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu));
  const uint32_t m1 = max(max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu), max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu));
  return max(m0, m1);
}

__global__ void __launch_bounds__(256) nv_amax_kernel(const uint4* __restrict__ x, int64_t n8, float* ts) {
  __shared__ uint32_t wmax[4];
  uint32_t a = 0;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * T < n8; i += 4 * T) {
    const uint4 w0 = x[i], w1 = x[i + T], w2 = x[i + 2 * T], w3 = x[i + 3 * T];
    a = max(a, max(max(bf16x8_absmax(w0), bf16x8_absmax(w1)), max(bf16x8_absmax(w2), bf16x8_absmax(w3))));
  }
  for (; i < n8; i += T) a = max(a, bf16x8_absmax(x[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<uint32_t*>(ts) + 1, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])) << 16);
}

// ---- axis 0 (Q, K): blocks along the contiguous last axis ----------------------------------
// One lane converts 8 consecutive elements (one 16-byte load); lanes 2k and 2k + 1 form a block.
__global__ void __launch_bounds__(256) nv_quantize_rows_kernel(const uint4* __restrict__ x, uint32_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales, float* ts, int64_t n8) {
  const uint32_t amax_t = reinterpret_cast<const uint32_t*>(ts)[1];
  const float G = nv_tensor_scale(amax_t);
  const float D6 = 6.0f * G;
  if (blockIdx.x == 0 && threadIdx.x == 0) ts[0] = G;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;    // even: pairs stay whole
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n8; g += stride) {
    const uint4 w = x[g];
    const float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                        bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, __float_as_uint(f[i]) & 0x7FFFFFFFu);
    am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false));   // partner lane
    const float S = e4m3_round(__uint_as_float(am) / D6);
    const float sigma = S > 0.0f ? S * G : __builtin_inff();    // S = 0: x / inf keeps the sign only
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f[i] / sigma;
    codes[g] = e2m1_pack8(v);
    if ((g & 1) == 0) scales[g >> 1] = (uint8_t)e4m3_byte(S);
  }
}

// ---- axis 1 (V): blocks along the sequence, written [bh][d][n] -------------------------------
// Grid (ceil(n / 128), d / 32, bh); a 128-token x 32-channel tile is staged in LDS ([token][channel],
// 17-dword rows), then thread t takes channel t % 32 and the 16-token block t / 32.
constexpr int NVC_TOK = 128, NVC_CH = 32, NVC_PITCH = 17;   // dwords per LDS row (16 + 1)
__global__ void __launch_bounds__(256) nv_quantize_cols_kernel(const uint32_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales, float* ts, int64_t n,
                                                               int64_t d) {
  __shared__ uint32_t tile[NVC_TOK * NVC_PITCH];
  const uint32_t amax_t = reinterpret_cast<const uint32_t*>(ts)[1];
  const float G = nv_tensor_scale(amax_t);
  const float D6 = 6.0f * G;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) ts[0] = G;
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * NVC_TOK, c0 = (int64_t)blockIdx.y * NVC_CH;
  const int ntok = (int)min((int64_t)NVC_TOK, n - t0);      // multiple of 16
  const uint32_t* xs = x + (bh * n + t0) * (d / 2) + c0 / 2;
  for (int k = tid; k < NVC_TOK * 4; k += 256) {
    const int r = k >> 2, cc = k & 3;                        // token, 8-channel chunk
    if (r < ntok) {
      const uint4 w = *reinterpret_cast<const uint4*>(xs + (int64_t)r * (d / 2) + 4 * cc);
      uint32_t* dst = tile + r * NVC_PITCH + 4 * cc;
      dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
    }
  }
  __syncthreads();
  const int ch = tid & 31, blk = tid >> 5;
  if (16 * blk >= ntok) return;
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t wv = tile[(16 * blk + i) * NVC_PITCH + (ch >> 1)];
    f[i] = (ch & 1) ? bf16_hi(wv) : bf16_lo(wv);
  }
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = max(am, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  const float S = e4m3_round(__uint_as_float(am) / D6);
  const float sigma = S > 0.0f ? S * G : __builtin_inff();
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = f[i] / sigma;
  const int64_t row = bh * d + c0 + ch;
  const int64_t tb = (t0 >> 4) + blk;                        // 16-token block
  *reinterpret_cast<uint2*>(codes + row * (n / 2) + 8 * tb) = make_uint2(e2m1_pack8(v), e2m1_pack8(v + 8));
  scales[row * (n / 16) + tb] = (uint8_t)e4m3_byte(S);
}

// ---- dequantize to fp16 (E2M1 * S, exact; the tensor scale is applied by the consumer) --------
// Flat over 8-element chunks (one code dword, half a scale byte, 16 output bytes).  Lane l of a
// wave takes chunks 64 j + l of the wave's 256, so that every load and store instruction of the
// wave covers one contiguous run.
__global__ void __launch_bounds__(256) nv_dequant_kernel(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                         uint4* __restrict__ out, int64_t chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); w * 256 < chunks; w += waves) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = w * 256 + 64 * j + lane;
      if (c < chunks) {
        const uint32_t cw = codes[c];
        const float s = e4m3_value(scales[c >> 1]);
        const v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
        const v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
        const v2f e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
        const v2f h = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
        out[c] = make_uint4(pk_f16_exact(a[0] * s, a[1] * s), pk_f16_exact(b[0] * s, b[1] * s),
                            pk_f16_exact(e[0] * s, e[1] * s), pk_f16_exact(h[0] * s, h[1] * s));
      }
    }
  }
}

// ---- forward ----------------------------------------------------------------------------------
// Workgroup = W waves of 32 query rows; key tiles of 64 staged in LDS by direct global -> LDS
// loads, two stages, one tile ahead.  S^T = K^ Q^T and O^T += V^T P~^T on the fp16 matrix core.
template <int D>
struct NvLds {
  static constexpr int KB = 0;                        // K^ fp16 [64 slots][D], swizzled chunks
  static constexpr int VT = KB + 64 * D * 2;          // V^T fp16 [D][64 keys], swizzled chunks
  static constexpr int BYTES = VT + D * 64 * 2;
};

template <int D, int W, bool CAUSAL>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
nv_fwd_kernel(NvFwdParams p) {
  using L = NvLds<D>;
  constexpr int DS_STEPS = D / 16;
  constexpr int CT = D / 32;
  constexpr int VC = D / 8;               // 16-B chunks per K^ fp16 row
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // work item: the workgroups of one head run on one XCD (blocks are dealt round-robin to the 8
  // XCDs); causal rows longest first
  const int64_t N = p.N;
  const int64_t nqt = N / (32 * W);
  const int64_t total = nqt * p.Hq * p.B;
  int64_t id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  const int64_t bh = id / nqt;
  int64_t qt = id - bh * nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int64_t b = bh / p.Hq, h = bh - b * p.Hq;
  const int64_t g = h / (p.Hq / p.Hkv);
  const int64_t bg = b * p.Hkv + g;
  const int64_t q0 = qt * 32 * W;
  const int64_t qw = q0 + 32 * wave;
  const int64_t row = qw + l32;

  const float gq = p.q_ts[0], gk = p.k_ts[0], gv = p.v_ts[0];
  const float snat = p.scale_nat * gq * gk;   // raw score -> natural-log units
  const float c = snat * kLog2e;              // raw score -> base-2 exponent

  // the wave's Q^ rows (fp16 B operand of S^T), fixed for the kernel
  v4i qf[DS_STEPS];
  {
    const uint16_t* qr = p.qb + (bh * N + row) * D;
#pragma unroll
    for (int s = 0; s < DS_STEPS; ++s) qf[s] = *reinterpret_cast<const v4i*>(qr + 16 * s + 8 * hi);
  }

  v16f acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v16f{};
  float mraw = -__builtin_inff();             // running max of the raw scores
  float mc = -__builtin_inff();               // mraw * c
  float lsum = 0.0f;                          // this lane's part of the row sum (E2M1 * S units)

  const int ntiles = (int)(CAUSAL ? ((q0 + 32 * W - 1) / 64 + 1) : (N / 64));
  const int last_active = CAUSAL ? (int)((qw + 31) / 64) : ntiles - 1;

  // staging jobs (one 64-lane LDS-DMA instruction, 1 KB, each): K^ rows, then V^T rows.  Each
  // lane's global source gives the LDS layout: slot s of the K^ tile holds key 32(s/32) +
  // row_key(s%32), so that register r of the S^T tile of half T in lane (l32, hi) is key
  // 32T + 16hi + r; chunks are XOR-swizzled per row.
  constexpr int NKB = 64 * D * 2 / 1024, NVT = D * 64 * 2 / 1024;
  constexpr int NJ = NKB + NVT;
  constexpr int JPW = NJ / W;
  static_assert(NJ % W == 0 && NKB % W == 0, "jobs per wave");
  const auto kb_rs = make_rsrc(p.kb + bg * N * D, N * D * 2);
  const auto vt_rs = make_rsrc(p.vt + bg * D * N, N * D * 2);
  auto goff_of = [&](int j) -> uint32_t {
    if (j < NKB) {
      const int cidx = 64 * j + lane, s = cidx / VC, cc = (cidx % VC) ^ swz_big(s, VC);
      return (32 * (s >> 5) + row_key(s & 31)) * (D * 2) + 16 * cc;
    }
    const int cidx = 64 * (j - NKB) + lane, ch = cidx >> 3, cc = (cidx & 7) ^ swz_big(ch, 8);
    return (uint32_t)ch * (uint32_t)(N * 2) + 16 * cc;
  };
  // with few jobs per wave the lane offsets are kept in registers, else recomputed per tile
  constexpr bool PRE = JPW <= 8;
  uint32_t job_goff[PRE ? JPW : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < JPW; ++i) job_goff[i] = goff_of(wave + W * i);
  }
  auto issue_tile = [&](int t, uint8_t* stage) __attribute__((always_inline)) {
    t = __builtin_amdgcn_readfirstlane(t);
#pragma unroll
    for (int i = 0; i < JPW; ++i) {
      const int j = wave + W * i;
      const uint32_t go = PRE ? job_goff[PRE ? i : 0] : goff_of(j);
      // jobs W i .. W i + W - 1 are all K^ or all V^T (NKB is a multiple of W)
      if (W * i < NKB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kb_rs, (__attribute__((address_space(3))) void*)(stage + L::KB + 1024 * j),
                                                 16, (int)go, t * (64 * D * 2), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vt_rs,
                                                 (__attribute__((address_space(3))) void*)(stage + L::VT + 1024 * (j - NKB)),
                                                 16, (int)go, t * (64 * 2), 0, 0);
    }
  };

  auto compute = [&](int t, const uint8_t* base) __attribute__((always_inline)) {
    v16f st[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int slot = 32 * T + l32;
      st[T] = v16f{};
#pragma unroll
      for (int s = 0; s < DS_STEPS; ++s) {
        const int cc = 2 * s + hi;
        const v4i a = *reinterpret_cast<const v4i*>(base + L::KB + slot * 2 * D + 16 * (cc ^ swz_big(slot, VC)));
        st[T] = mfma_f16(a, qf[s], st[T]);
      }
      if (CAUSAL && ((int64_t)t * 64 + 63 > qw)) {
        const int jrel = (int)(row - (int64_t)t * 64) - 32 * T - 16 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r > jrel) st[T][r] = -__builtin_inff();
      }
    }
    // block maxima (a lane's 16 keys of a half are one 16-key block) and the row max
    float bm[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      float x = st[T][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, st[T][r]);
      bm[T] = x;
    }
    float mt = fmaxf(bm[0], bm[1]);
    {
      // lanes l and l + 32 hold the two halves of a row: after the swap one result holds the
      // lane's own value and the other the partner's
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mraw_new = fmaxf(mraw, mt);
    const float mc_new = mraw_new * c;
    const float mc_prev = mc;
    const bool raised = mraw_new != mraw;         // else alpha = exp2(0) = 1: nothing to rescale
    mraw = mraw_new;
    mc = mc_new;
    if (__builtin_amdgcn_ballot_w64(raised)) {
      const float alpha = __builtin_amdgcn_exp2f(mc_prev - mc_new);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ct][r] *= alpha;
      lsum *= alpha;
    }
    // P~ per block: S = E4M3(max p * 448), P~ 2688 = E2M1(v) S with v = p 2688 / S (fp16, exact).
    // v = 2^(s c - mc + log2(2688 / S)): the division by S rides on the exponential.  With
    // S = 2^k mu (mu in [1, 2)), the decode to fp16 applies 2^k (the convert takes only the
    // exponent of its scale operand) and one packed multiply applies mu to two values.
    uint32_t pw[2][8];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const float bp = __builtin_amdgcn_exp2f(__builtin_fmaf(bm[T], c, -mc));
      const float S = e4m3_round(bp * 448.0f);
      const float sh = S > 0.0f ? mc - (kLog2NvDiv - __builtin_amdgcn_logf(S)) : __builtin_inff();
      const _Float16 mu = (_Float16)__uint_as_float((__float_as_uint(S) & 0x007FFFFFu) | 0x3F800000u);
      const v2h mu2 = {mu, mu};
      const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[T][r], c, -sh));
      const uint32_t c0 = e2m1_pack8(v), c1 = e2m1_pack8(v + 8);
      static_for<8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const v2h x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q < 4 ? c0 : c1, S, q & 3) * mu2;
        lsum = __builtin_amdgcn_fdot2(x, ones, lsum, false);
        pw[T][q] = __builtin_bit_cast(uint32_t, x);
      });
    }
    // O^T += V^T P~^T: k-step s2 of half T takes keys 32T + 16hi + 8s2 + [0, 8) (registers 8s2..)
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const v4i bsv = v4i{(int)pw[T][4 * s2], (int)pw[T][4 * s2 + 1], (int)pw[T][4 * s2 + 2], (int)pw[T][4 * s2 + 3]};
        const int cc = 4 * T + 2 * hi + s2;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int ch = 32 * ct + l32;
          const v4i a = *reinterpret_cast<const v4i*>(base + L::VT + ch * 128 + 16 * (cc ^ swz_big(ch, 8)));
          acc[ct] = mfma_f16(a, bsv, acc[ct]);
        }
      }
  };

  // step t: prefetch tile t + 1 into the other stage, compute tile t; the barrier that ends the
  // step publishes tile t + 1 (each wave first waits for its own DMAs) and frees stage t.
  issue_tile(0, smem);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  auto step = [&](int t, auto stc) __attribute__((always_inline)) {
    constexpr int sg = decltype(stc)::value;
    if (t + 1 < ntiles) issue_tile(t + 1, smem + (sg ^ 1) * L::BYTES);
    if (t <= last_active) compute(t, smem + sg * L::BYTES);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 >= ntiles) break;
    step(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = G_V acc / l; lane holds query `row`, channels 32ct + 8a + 4hi + [0, 4) ----
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float sc = lsum > 0.0f ? gv / lsum : 0.0f;
  uint16_t* orow = p.o + (bh * N + row) * D;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * ct + 8 * a + 4 * hi;
      *reinterpret_cast<uint2*>(orow + ch) = make_uint2(pk_bf16(sc * acc[ct][4 * a], sc * acc[ct][4 * a + 1]),
                                                        pk_bf16(sc * acc[ct][4 * a + 2], sc * acc[ct][4 * a + 3]));
    }
  if (hi == 0) {
    p.m[bh * N + row] = mraw * snat;
    p.l[bh * N + row] = lsum * (1.0f / kNvDiv);
  }
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

unsigned grid_for(int64_t units) {
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

template <int D, bool CAUSAL>
hipError_t launch_nv_fwd_d(const NvFwdParams& p, hipStream_t stream) {
  if (p.N % 256 == 0)
    hipLaunchKernelGGL((nv_fwd_kernel<D, 8, CAUSAL>), dim3((unsigned)((p.N / 256) * p.Hq * p.B)), dim3(512), 0, stream, p);
  else if (p.N % 128 == 0)
    hipLaunchKernelGGL((nv_fwd_kernel<D, 4, CAUSAL>), dim3((unsigned)((p.N / 128) * p.Hq * p.B)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((nv_fwd_kernel<D, 2, CAUSAL>), dim3((unsigned)((p.N / 64) * p.Hq * p.B)), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_nv_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int axis, void* codes, void* scales,
                              float* ts, hipStream_t stream) {
  const int64_t n8 = bh * n * d / 8;
  hipLaunchKernelGGL(nv_amax_clear_kernel, dim3(1), dim3(1), 0, stream, ts);
  hipLaunchKernelGGL(nv_amax_kernel, dim3(min(grid_for((n8 + 3) / 4), 2048u)), dim3(256), 0, stream, (const uint4*)x,
                     n8, ts);
  if (axis == 0) {
    hipLaunchKernelGGL(nv_quantize_rows_kernel, dim3(grid_for(n8)), dim3(256), 0, stream, (const uint4*)x,
                       (uint32_t*)codes, (uint8_t*)scales, ts, n8);
  } else {
    dim3 grid((unsigned)((n + NVC_TOK - 1) / NVC_TOK), (unsigned)(d / NVC_CH), (unsigned)bh);
    hipLaunchKernelGGL(nv_quantize_cols_kernel, grid, dim3(256), 0, stream, (const uint32_t*)x, (uint8_t*)codes,
                       (uint8_t*)scales, ts, n, d);
  }
  return hipGetLastError();
}

NvWorkspace nv_fwd_workspace_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
  NvWorkspace w;
  w.qb = 0;
  w.kb = w.qb + align256(B * Hq * N * d * 2);
  w.vt = w.kb + align256(B * Hkv * N * d * 2);
  w.total = w.vt + align256(B * Hkv * N * d * 2);
  return w;
}

hipError_t launch_nv_fwd(const NvFwdParams& p, const void* q_codes, const void* q_scales, const void* k_codes,
                         const void* k_scales, const void* v_codes, const void* v_scales, int d, bool causal,
                         hipStream_t stream) {
  struct Job { const void* c; const void* s; const uint16_t* out; int64_t chunks; };
  const Job jobs[3] = {{q_codes, q_scales, p.qb, p.B * p.Hq * p.N * d / 8},
                       {k_codes, k_scales, p.kb, p.B * p.Hkv * p.N * d / 8},
                       {v_codes, v_scales, p.vt, p.B * p.Hkv * p.N * d / 8}};
  for (const Job& j : jobs)
    hipLaunchKernelGGL(nv_dequant_kernel, dim3(grid_for((j.chunks + 3) / 4)), dim3(256), 0, stream, (const uint32_t*)j.c,
                       (const uint8_t*)j.s, (uint4*)const_cast<uint16_t*>(j.out), j.chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d == 128) return causal ? launch_nv_fwd_d<128, true>(p, stream) : launch_nv_fwd_d<128, false>(p, stream);
  return causal ? launch_nv_fwd_d<64, true>(p, stream) : launch_nv_fwd_d<64, false>(p, stream);
}

}  // namespace attnfp4
