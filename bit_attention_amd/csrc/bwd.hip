// Attn-QAT backward with FP4 recomputation of the scores, for gfx950.
//
// What is computed (Attn-QAT abstract: (1) the backward recomputes the attention scores with the
// same low-precision QK^T as the forward, (2) the D term of the FlashAttention gradient is taken
// from the FP4 forward's own output rather than assuming O = PV in high precision).  With the
// forward's final row max m and row sum l, and gradients passing straight through the quantizers:
//   D_i  = sum_c dO_ic O_ic                                (fp32)
//   S^   = Q^ K^T * scale  (scaled FP4 MFMA, as in the forward)
//   p    = exp(S^ - m),  P = p / l,  A = MXFP4(p) / l      (P requantized per 32-key block)
//   dV   = A^T dO,  dP = dO V^T,  dS = P o (dP - D)
//   dQ   = scale dS K^,  dK = scale dS^T Q^               (bf16 MFMA, fp32 accumulation)
//
// Kernels (one launch each, all on the caller's stream):
//  1. rows: D, m log2(e) and 1/l per query row.
//  2. transposes: bf16 copies of the dequantized operands in the layouts the bf16 MFMAs read
//     (V^ as [N, d]; K^, Q^ as [d, N]; FP4 * 2^e is exact in bf16), and dO^T [d, N] with each
//     query's 1/l folded in (dO * (1/l) rounded to bf16 once).
//  3. dK/dV: a workgroup owns 16W keys (32-key pairs of waves) and walks all query rows of the
//     KV head's query heads in tiles of 64.  S^T and dP^T are computed with one lane per query so
//     that the 32-key P blocks sit in one lane pair, P~ is requantized in registers exactly as in
//     the forward, and P~ (exact in bf16; its 1/l rides on dO^T) and dS pass through LDS to feed
//     the dV^T = (dO diag(1/l))^T P~ and dK^T = Q^T dS products.
//  4. dQ: a workgroup owns 32W query rows and walks the keys in tiles of 64:
//     dQ^T = K^T dS^T with dS^T taken straight from registers.  No atomics: dQ, dK, dV are each
//     written once, so the backward is deterministic.
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"

namespace attnfp4 {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
__device__ __forceinline__ v8i widen(v4i x) { return v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }

// XOR swizzle of the 16-byte chunks of an FP4 code row in LDS (64 B = 4 chunks at d = 128, 32 B =
// 2 chunks at d = 64), so that 16 lanes reading one logical chunk of 16 consecutive rows hit 16
// distinct 4-bank groups.
__device__ __forceinline__ int swz_code(int row, int nchunks) {
  return nchunks == 4 ? (((row >> 1) ^ (row >> 2)) & 3) : ((row >> 3) & 1);
}

// ---------------------------------------------------------------------------------------------
// 1. per-row constants
// 16 lanes per row; rows = B*Hq*N is a multiple of 16.
__global__ void __launch_bounds__(256) bwd_rows_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ m,
                                                       const float* __restrict__ l, float* __restrict__ rowc,
                                                       int64_t rows, int d,
                                                       const uint8_t* __restrict__ q_codes = nullptr,
                                                       const uint8_t* __restrict__ q_scales = nullptr,
                                                       uint16_t* __restrict__ qb = nullptr,
                                                       uint16_t* __restrict__ dos = nullptr) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  if (r >= rows) return;
  const int per = d / 16;                       // 8 (d = 128) or 4 (d = 64) elements per lane
  const uint16_t* orow = o + r * d + sub * per;
  const uint16_t* grow = dout + r * d + sub * per;
  // the lane's O and dO elements in one load each (16 bytes at d = 128, 8 at d = 64)
  uint32_t ow[4] = {0, 0, 0, 0}, gw[4] = {0, 0, 0, 0};
  if (per == 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(orow), g = *reinterpret_cast<const uint4*>(grow);
    ow[0] = a.x; ow[1] = a.y; ow[2] = a.z; ow[3] = a.w;
    gw[0] = g.x; gw[1] = g.y; gw[2] = g.z; gw[3] = g.w;
  } else {
    const uint2 a = *reinterpret_cast<const uint2*>(orow), g = *reinterpret_cast<const uint2*>(grow);
    ow[0] = a.x; ow[1] = a.y;
    gw[0] = g.x; gw[1] = g.y;
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {                 // the zero padding at d = 64 adds nothing
    acc = __builtin_fmaf(bf16_lo(ow[i]), bf16_lo(gw[i]), acc);
    acc = __builtin_fmaf(bf16_hi(ow[i]), bf16_hi(gw[i]), acc);
  }
  acc += __shfl_xor(acc, 1, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 8, 16);
  const float il = 1.0f / l[r];
  if (sub == 0) *reinterpret_cast<float4*>(rowc + 4 * r) = make_float4(m[r] * kLog2e, il, acc, acc * il);
  if (dos != nullptr) {                         // dO / l, rounded to bf16 once (d = 128)
    const uint32_t* w = gw;
    uint4 out;
    out.x = pk_bf16(bf16_lo(w[0]) * il, bf16_hi(w[0]) * il);
    out.y = pk_bf16(bf16_lo(w[1]) * il, bf16_hi(w[1]) * il);
    out.z = pk_bf16(bf16_lo(w[2]) * il, bf16_hi(w[2]) * il);
    out.w = pk_bf16(bf16_lo(w[3]) * il, bf16_hi(w[3]) * il);
    *reinterpret_cast<uint4*>(dos + r * d + sub * 8) = out;
  }
  if (qb != nullptr) {                          // Q^ dequantized to bf16 (exact), d = 128
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(q_codes + r * (d / 2) + sub * 4);
    const int e = (int)q_scales[r * (d / 32) + sub / 4] - 127;
    const v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
    const v2f bb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
    const v2f cc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
    const v2f dd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
    const float v[8] = {a[0], a[1], bb[0], bb[1], cc[0], cc[1], dd[0], dd[1]};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = __float_as_uint(__builtin_ldexpf(v[i], e)) >> 16;   // exact in bf16
    *reinterpret_cast<uint4*>(qb + r * d + sub * 8) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  }
}

// ---------------------------------------------------------------------------------------------
// 2. 64x64 tile transpose to bf16: src logical [batch][R][C] -> dst [batch][C][R].
//    FP4: src = packed E2M1 codes with E8M0 scales along C (dequantized exactly), row-major
//    ([R][C/2] and [R][C/32]) or, with BLOCK_MAJOR, the V^ layout ([C/32][R][16], [C/32][R]);
//    otherwise src = bf16 [R][C], each row multiplied by rscale[4 row] (when given: the 1/l entry
//    of the per-row constants) and rounded to bf16 once.
template <bool FP4, bool BLOCK_MAJOR = false>
__global__ void __launch_bounds__(256) bwd_transpose_kernel(const uint8_t* __restrict__ src,
                                                            const uint8_t* __restrict__ scl,
                                                            uint16_t* __restrict__ dst, int64_t R, int64_t C,
                                                            const float* __restrict__ rscale = nullptr) {
  __shared__ uint16_t tile[64][66];
  const int tid = threadIdx.x;
  const int64_t bz = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  {
    const int r = tid >> 2, cq = (tid & 3) * 16;
    const int64_t row = bz * R + r0 + r;
    if (FP4) {
      const int64_t blk = (c0 + cq) / 32;   // block-major: [batch][C/32][R][16 bytes]
      const uint2 w = BLOCK_MAJOR
                          ? *reinterpret_cast<const uint2*>(src + bz * (R * C / 2) + (blk * R + r0 + r) * 16 + ((cq & 31) >> 1))
                          : *reinterpret_cast<const uint2*>(src + (row * C + c0 + cq) / 2);
      const int e = (int)(BLOCK_MAJOR ? scl[bz * (R * C / 32) + blk * R + r0 + r] : scl[row * (C / 32) + blk]) - 127;
      const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww[q], 1.0f, 0);
        v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww[q], 1.0f, 1);
        v2f c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww[q], 1.0f, 2);
        v2f dd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww[q], 1.0f, 3);
        const float v[8] = {a[0], a[1], b[0], b[1], c[0], c[1], dd[0], dd[1]};
#pragma unroll
        for (int i = 0; i < 8; ++i)   // E2M1 * 2^e is exact in fp32 and in bf16
          tile[r][cq + 8 * q + i] = (uint16_t)(__float_as_uint(__builtin_ldexpf(v[i], e)) >> 16);
      }
    } else {
      const uint4* s = reinterpret_cast<const uint4*>(src + (row * C + c0 + cq) * 2);
      const uint4 a = s[0], b = s[1];
      uint32_t ww[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      if (rscale != nullptr) {
        const float f = rscale[4 * row];
#pragma unroll
        for (int i = 0; i < 8; ++i) ww[i] = pk_bf16(bf16_lo(ww[i]) * f, bf16_hi(ww[i]) * f);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tile[r][cq + 2 * i] = (uint16_t)(ww[i] & 0xFFFF);
        tile[r][cq + 2 * i + 1] = (uint16_t)(ww[i] >> 16);
      }
    }
  }
  __syncthreads();
  {
    const int c = tid >> 2, rq = (tid & 3) * 16;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (uint32_t)tile[rq + 2 * i][c] | ((uint32_t)tile[rq + 2 * i + 1][c] << 16);
    uint4* d = reinterpret_cast<uint4*>(dst + ((bz * C + c0 + c) * R + r0 + rq));
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// ---------------------------------------------------------------------------------------------
// The P~ block scale of one 32-key block in the backward.  The block's largest p is
// exp2(bmax c - m log2 e); for the block holding the row's maximum it is 1 in exact arithmetic
// (m is that maximum), but the fp32 rounding of the saved m can leave it a hair below 1, which
// would halve the scale and saturate the maximum to 0.75.  Values within a few ulps of the row
// maximum are therefore taken as exactly the maximum.  Exponents below -126 are clamped (affects
// only P < 2^-124).
__device__ __forceinline__ int p_scale_byte(float tb, float mq) {
  const float tol = fmaxf(__builtin_fabsf(mq) * 0x1p-20f, 0x1p-22f);
  const float pm = tb > -tol ? 1.0f : __builtin_amdgcn_exp2f(tb);
  return max((int)(__float_as_uint(pm) >> 23) - 2, 1);
}

// Four transposing LDS loads (ds_read_b64_tr_b16) and the wait for them, in one statement: the
// results are complete when it ends.  (The builtin form makes the compiler wait for every direct
// global-to-LDS load in flight first, which would serialise the staging of the next tiles.)
__device__ __forceinline__ void lds_read_tr4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, v2i& r0, v2i& r1,
                                             v2i& r2, v2i& r3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3));
}

// ---------------------------------------------------------------------------------------------
// 3. dK / dV.  Workgroup = W waves; wave w: pair p = w/2 owns keys k0 + 32p + [0, 32), half = w%2
// takes query sub-tile `half` in the elementwise phase and channel half `half` in the products.
// The query tile's operands are staged by direct global -> LDS loads in two groups, each double
// buffered: group A (Q^ codes and scales, the row constants, dO) is read by the elementwise phase,
// group B (dO^T, Q^T) by the products.  The products phase of tile n issues group A of tile n + 2
// and group B of tile n + 1, so that every load has about a whole tile to land before the one
// wait per tile (ahead of the products).  A = P~/l and dS pass from the elementwise phase to the
// products query-major ([64 q][KEYS], 16-byte chunks swizzled by the row): a lane writes its 16
// keys of one query as two 16-byte stores, and the products read them back as [key][query]
// operands with the transposing LDS load.
template <int D, int W>
struct DkdvLds {
  static constexpr int KEYS = 16 * W;                 // 32 keys per pair of waves
  static constexpr int QC = 0;                        // A: Q^ codes [64 q][D/2]
  static constexpr int QS = QC + 64 * D / 2;          // A: Q^ scales [64 q] dwords
  static constexpr int ROWS = QS + 64 * 4;            // A: (mq, il, D, 0) [64 q] float4
  static constexpr int DO = ROWS + 64 * 16;           // A: dO bf16 [64 q][D], swizzled chunks
  static constexpr int A_BYTES = DO + 64 * D * 2;
  static constexpr int DOT = 0;                       // B: dO^T bf16 [D][64 q], swizzled chunks
  static constexpr int QT = DOT + D * 64 * 2;         // B: Q^T bf16 [D][64 q], swizzled chunks
  static constexpr int B_BYTES = QT + D * 64 * 2;
  static constexpr int A0 = 0;                        // two group-A buffers, then two group-B
  static constexpr int B0 = 2 * A_BYTES;
  static constexpr int PS = B0 + 2 * B_BYTES;         // A = P~/l bf16 [64 q][KEYS], swizzled chunks
  static constexpr int DS = PS + 64 * KEYS * 2;       // dS bf16 [64 q][KEYS]
  static constexpr int BYTES = DS + 64 * KEYS * 2;
  static constexpr int NCH = KEYS / 8;                // 16-byte chunks per scratch row
  static_assert(NCH == 8 || NCH == 16, "scratch swizzle");
  // byte offset of (query row q, key chunk c) in the scratch.  The chunk is XORed with bits of the
  // row so that both access patterns spread over all banks: a lane's two 16-byte stores (32 rows
  // of one chunk per instruction) and the transposing loads (4 consecutive rows x 4 chunks per
  // 16 lanes, two such row groups 8 apart per instruction).
  static __device__ __forceinline__ int chunk(int q, int c) {
    const int x = NCH == 16 ? (((q & 3) << 2) | ((q >> 2) & 3)) : (((q & 3) << 1) | ((q >> 2) & 1));
    return q * (KEYS * 2) + 16 * (c ^ x);
  }
};

template <int D, int W, bool CAUSAL>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdParams p) {
  using L = DkdvLds<D, W>;
  constexpr int KS_STEPS = D / 64;        // FP4 k-steps of S^T
  constexpr int DS_STEPS = D / 16;        // bf16 k-steps of dP^T
  constexpr int CH = D / 2;               // channels accumulated per wave
  constexpr int CT = CH / 32;             // 32-channel tiles per wave
  constexpr int RC = D / 8;               // 16-B chunks per dO row
  constexpr int KCH = D / 32;             // 16-B chunks per Q^ code row
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int pair = wave >> 1, half = wave & 1;

  const int64_t N = p.N;
  const int64_t nkt = N / L::KEYS;
  const int64_t bg = blockIdx.x / nkt;            // b * Hkv + g
  const int64_t k0 = (blockIdx.x - bg * nkt) * L::KEYS;
  const int64_t b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int64_t group = p.Hq / p.Hkv;
  const int64_t kp = k0 + 32 * pair;              // the pair's first key
  const float c = p.c;

  // ---- constant operands of this wave: K^ (FP4) and V^ (bf16) rows of the pair's 32 keys, in the
  //      row order that makes lane l hold keys kp + 16(l/32) + r in S^T / dP^T register r ----
  const int64_t krow = kp + row_key(l32);
  v4i ka[KS_STEPS];
  const uint8_t* kr = p.k_codes + (bg * N + krow) * (D / 2);
#pragma unroll
  for (int ks = 0; ks < KS_STEPS; ++ks) ka[ks] = *reinterpret_cast<const v4i*>(kr + 16 * hi + 32 * ks);
  const uint8_t* ksr = p.k_scales + (bg * N + krow) * (D / 32);
  const int ksc = (D == 128) ? (int)(ksr[hi] | (ksr[2 + hi] << 16)) : (int)ksr[hi];
  v4i va[DS_STEPS];
  const uint16_t* vr = p.vb + (bg * N + krow) * D;
#pragma unroll
  for (int s = 0; s < DS_STEPS; ++s) va[s] = *reinterpret_cast<const v4i*>(vr + 16 * s + 8 * hi);

  v16f dv[CT], dk[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    dv[ct] = v16f{};
    dk[ct] = v16f{};
  }

  // ---- staging jobs (one 64-lane LDS-DMA instruction each) ----
  // group A: dO (1-KB pieces), Q^ codes (1-KB pieces), the Q^ scales and the per-row constants;
  // group B: dO^T, Q^T.  Job j of a group is issued by wave j % W in slot j / W (the last job
  // repeated where the list runs out: an identical rewrite).  A slot whose jobs are all of one kind
  // is emitted without a branch, a mixed one with at most two wave-uniform compares.  The query
  // heads of this KV head are contiguous, so one resource per tensor covers them; the tile's
  // (head, row) offset goes in the scalar offset.
  constexpr int NQC = 64 * D / 2 / 1024, NDO = 64 * D * 2 / 1024;
  constexpr int NA = NDO + NQC + 2, NB = 2 * (D * 64 * 2 / 1024);
  constexpr int JA = (NA + W - 1) / W, JB = (NB + W - 1) / W;
  const int64_t hq0 = b * p.Hq + g * group;       // first query head of this KV head
  const auto qc_rs = make_rsrc(p.q_codes + hq0 * N * (D / 2), group * N * (D / 2));
  const auto qs_rs = make_rsrc(p.q_scales + hq0 * N * (D / 32), group * N * (D / 32));
  const auto do_rs = make_rsrc(p.dout + hq0 * N * D, group * N * D * 2);
  const auto rc_rs = make_rsrc(p.rowc + hq0 * N * 4, group * N * 16);
  const auto dot_rs = make_rsrc(p.dot + hq0 * D * N, group * D * N * 2);
  const auto qt_rs = make_rsrc(p.qt + hq0 * D * N, group * D * N * 2);
  // kinds: 0 dO, 1 Q^ codes, 2 Q^ scales, 3 row constants | 4 dO^T, 5 Q^T
  auto kind_a = [](int j) constexpr { return j < NDO ? 0 : j < NDO + NQC ? 1 : j == NDO + NQC ? 2 : 3; };
  auto kind_b = [](int j) constexpr { return j < NB / 2 ? 4 : 5; };
  auto goff_of = [&](int kind, int j) -> uint32_t {   // lane's global byte offset within the tile
    if (kind == 0) {
      const int cidx = 64 * j + lane, q = cidx / RC, cc = (cidx % RC) ^ swz_big(q, RC);
      return q * (D * 2) + 16 * cc;
    }
    if (kind == 1) {                                   // Q^ codes, chunks swizzled by row
      const int cidx = 64 * (j - NDO) + lane, q = cidx / KCH, cc = (cidx % KCH) ^ swz_code(q, KCH);
      return q * (D / 2) + 16 * cc;
    }
    if (kind == 2) return lane * (D / 32);
    if (kind == 3) return 16 * lane;
    const int cidx = 64 * (kind == 4 ? j : j - NB / 2) + lane, ch = cidx >> 3, cc = (cidx & 7) ^ swz_big(ch, 8);
    return (uint32_t)ch * (uint32_t)(N * 2) + 16 * cc;
  };
  auto dst_of = [](int kind, int j) -> int {   // within the group's buffer
    return kind == 0 ? L::DO + 1024 * j : kind == 1 ? L::QC + 1024 * (j - NDO) : kind == 2 ? L::QS : kind == 3 ? L::ROWS
         : kind == 4 ? L::DOT + 1024 * j : L::QT + 1024 * (j - NB / 2);
  };
  uint32_t goff_a[JA], goff_b[JB];
#pragma unroll
  for (int i = 0; i < JA; ++i) { const int j = min(wave + W * i, NA - 1); goff_a[i] = goff_of(kind_a(j), j); }
#pragma unroll
  for (int i = 0; i < JB; ++i) { const int j = min(wave + W * i, NB - 1); goff_b[i] = goff_of(kind_b(j), j); }
  // one job of a compile-time kind; r = the tile's first row of [head][N], tcol = its first element
  // of [head][D][N] (both wave-uniform)
  auto issue_kind = [&](auto kc, int j, uint32_t goff, int r, int tcol, int buf) __attribute__((always_inline)) {
    constexpr int kind = decltype(kc)::value;
    const int base = kind <= 3 ? L::A0 + buf * L::A_BYTES : L::B0 + buf * L::B_BYTES;
    auto* dst = (__attribute__((address_space(3))) void*)(smem + base + dst_of(kind, j));   // LDS-DMA target
    if constexpr (kind == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(do_rs, dst, 16, (int)goff, r * (D * 2), 0, 0);
    else if constexpr (kind == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(qc_rs, dst, 16, (int)goff, r * (D / 2), 0, 0);
    else if constexpr (kind == 2) {   // d/32 bytes per row
      if constexpr (D == 128) __builtin_amdgcn_raw_ptr_buffer_load_lds(qs_rs, dst, 4, (int)goff, r * (D / 32), 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(qs_rs, dst, 2, (int)goff, r * (D / 32), 0, 0);
    } else if constexpr (kind == 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(rc_rs, dst, 16, (int)goff, r * 16, 0, 0);
    else if constexpr (kind == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(dot_rs, dst, 16, (int)goff, tcol * 2, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(qt_rs, dst, 16, (int)goff, tcol * 2, 0, 0);
  };
  // slot i of a group: the kinds of its jobs span [klo, khi] (known at compile time)
  auto issue_slot = [&](auto klo_c, auto khi_c, int kind, int j, uint32_t goff, int r, int tcol, int buf)
      __attribute__((always_inline)) {
    constexpr int klo = decltype(klo_c)::value, khi = decltype(khi_c)::value;
    static_assert(khi - klo <= 2, "kinds per slot");
    using K0 = std::integral_constant<int, klo>;
    using K1 = std::integral_constant<int, (klo + 1 < khi ? klo + 1 : khi)>;
    using K2 = std::integral_constant<int, khi>;
    if constexpr (klo == khi) issue_kind(K0{}, j, goff, r, tcol, buf);
    else if (kind == klo) issue_kind(K0{}, j, goff, r, tcol, buf);
    else if (khi - klo >= 2 && kind == klo + 1) issue_kind(K1{}, j, goff, r, tcol, buf);
    else issue_kind(K2{}, j, goff, r, tcol, buf);
  };
  auto issue_a = [&](int r, int buf) __attribute__((always_inline)) {
    static_for<JA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int jlo = W * i < NA - 1 ? W * i : NA - 1, jhi = W * i + W - 1 < NA - 1 ? W * i + W - 1 : NA - 1;
      const int j = min(wave + W * i, NA - 1);
      issue_slot(std::integral_constant<int, kind_a(jlo)>{}, std::integral_constant<int, kind_a(jhi)>{}, kind_a(j), j,
                 goff_a[i], r, 0, buf);
    });
  };
  auto issue_b = [&](int tcol, int buf) __attribute__((always_inline)) {
    static_for<JB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int jlo = W * i < NB - 1 ? W * i : NB - 1, jhi = W * i + W - 1 < NB - 1 ? W * i + W - 1 : NB - 1;
      const int j = min(wave + W * i, NB - 1);
      issue_slot(std::integral_constant<int, kind_b(jlo)>{}, std::integral_constant<int, kind_b(jhi)>{}, kind_b(j), j,
                 goff_b[i], 0, tcol, buf);
    });
  };

  // ---- tiles: the query heads of the group, and per head the query tiles that see any key ----
  // (all wave-uniform 32-bit scalars: group * D * N * 2 < 2^31 is checked at the boundary)
  const int j_first = CAUSAL ? (int)(k0 / 64) : 0;   // query tiles below the keys see none of them
  const int nj = (int)(N / 64) - j_first;
  const int ntile = (int)group * nj;
  // query tile n as (head of the group, tile j of the head): the tiles of a head are consecutive
  auto next = [&](int& h_, int& j_) __attribute__((always_inline)) {
    if (++j_ == nj) { j_ = 0; ++h_; }
  };
  auto row_of = [&](int h_, int j_) __attribute__((always_inline)) {        // first row of [head][N]
    return __builtin_amdgcn_readfirstlane(h_ * (int)N + (j_first + j_) * 64);
  };
  auto tcol_of = [&](int h_, int j_) __attribute__((always_inline)) {       // first element of [head][D][N]
    return __builtin_amdgcn_readfirstlane(h_ * D * (int)N + (j_first + j_) * 64);
  };
  int jj = 0;                                      // tile n (its row within the head)
  int hn = 0, jn = 0;                              // tile n + 1
  next(hn, jn);
  issue_a(row_of(0, 0), 0);
  issue_b(tcol_of(0, 0), 0);
  if (ntile > 1) issue_a(row_of(hn, jn), 1);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // one tile; the buffer index is a compile-time constant (the loop below is unrolled by two) so
  // that the compiler sees which LDS bytes the direct loads write and adds no waits of its own
  auto tile = [&](auto bufc, int n) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int q0 = (j_first + jj) * 64;
    int h2 = hn, j2 = jn;                           // tile n + 2
    next(h2, j2);
    const uint8_t* sa = smem + L::A0 + buf * L::A_BYTES;
    const uint8_t* sb = smem + L::B0 + buf * L::B_BYTES;

    // ---- elementwise phase: keys kp + [0,32) x queries q0 + 32 half + [0,32) ----
    {
      const int ql = 32 * half + l32;                  // this lane's query within the tile
      const int64_t qrow = q0 + ql;
      // S^T = K^ Q^T (FP4)
      const uint8_t* qcl = sa + L::QC + ql * (D / 2);
      const int qx = swz_code(ql, KCH);
      const uint32_t qsw = *reinterpret_cast<const uint32_t*>(sa + L::QS + 4 * ql);
      const int qsc = (int)(qsw >> (8 * hi));
      v16f st = v16f{};
      st = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka[0]), widen(*reinterpret_cast<const v4i*>(qcl + 16 * (hi ^ qx))),
                                                          st, 4, 4, 0, ksc, 0, qsc);
      if (KS_STEPS == 2)
        st = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            widen(ka[KS_STEPS - 1]), widen(*reinterpret_cast<const v4i*>(qcl + 16 * ((hi + 2) ^ qx))), st, 4, 4, 2, ksc, 2, qsc);
      // dP^T = V^ dO^T (bf16)
      v16f dp = v16f{};
#pragma unroll
      for (int s = 0; s < DS_STEPS; ++s) {
        const int cc = 2 * s + hi;
        const v4i bo = *reinterpret_cast<const v4i*>(sa + L::DO + ql * 2 * D + 16 * (cc ^ swz_big(ql, RC)));
        dp = mfma_bf16(va[s], bo, dp);
      }
      const float4 rc = reinterpret_cast<const float4*>(sa + L::ROWS)[ql];
      const float mq = rc.x, il = rc.y, dd = rc.z;
      // register r holds key kp + 16 hi + r
      if (CAUSAL) {
        const int jrel = (int)(qrow - kp) - 16 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r > jrel) st[r] = -__builtin_inff();
      }
      float mx = st[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      const float bmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const int sbyte = p_scale_byte(__builtin_fmaf(bmax, c, -mq), mq);
      const float sc = __uint_as_float((uint32_t)sbyte << 23);
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c, -mq));
      uint32_t aw[8], sw8[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t u = 0;
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, pr[4 * q], pr[4 * q + 1], sc, 0);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, pr[4 * q + 2], pr[4 * q + 3], sc, 1);
        // A = P~ itself (exact in bf16); the 1/l of its query is carried by the dO^T operand
        aw[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, sc, 0));
        aw[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, sc, 1));
        float ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ds[i] = pr[4 * q + i] * il * (dp[4 * q + i] - dd);
        sw8[2 * q] = pk_bf16(ds[0], ds[1]);
        sw8[2 * q + 1] = pk_bf16(ds[2], ds[3]);
      }
      // query-major scratch: row ql, keys 32 pair + 16 hi + [0, 16) = chunks 4 pair + 2 hi + {0, 1}
      const int c0 = 4 * pair + 2 * hi;
      *reinterpret_cast<v4i*>(smem + L::PS + L::chunk(ql, c0)) = v4i{(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3]};
      *reinterpret_cast<v4i*>(smem + L::PS + L::chunk(ql, c0 + 1)) = v4i{(int)aw[4], (int)aw[5], (int)aw[6], (int)aw[7]};
      *reinterpret_cast<v4i*>(smem + L::DS + L::chunk(ql, c0)) = v4i{(int)sw8[0], (int)sw8[1], (int)sw8[2], (int)sw8[3]};
      *reinterpret_cast<v4i*>(smem + L::DS + L::chunk(ql, c0 + 1)) = v4i{(int)sw8[4], (int)sw8[5], (int)sw8[6], (int)sw8[7]};
    }
    // group B of this tile (and group A of the next) has landed; the scratch is written
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- products: dV^T += dO^T A, dK^T += Q^T dS over the tile's 64 queries ----
    {
      // transposing reads of the query-major scratch: in each 16-lane group, lane i supplies
      // keys kb + 4 (i % 4) + [0, 4) of query row qb + i / 4, and lane j receives key kb + j of
      // rows qb .. qb + 3; the group's keys kb = 32 pair + 16 (lane / 16 % 2), its rows start at
      // 16 s + 8 hi + 4 t
      const int gi = lane & 15;
      const int kst = 32 * pair + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
      const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
      auto tr_addr = [&](int region, int qrw) -> uint32_t {
        return lds0 + (uint32_t)(region + L::chunk(qrw, kst >> 3) + 2 * (kst & 7));
      };
      // group A of tile n + 2 (into this tile's A buffer, read by the elementwise phase that has
      // ended) and group B of tile n + 1 (into the other B buffer, free since tile n - 1)
      if (n + 2 < ntile) issue_a(row_of(h2, j2), buf);
      if (n + 1 < ntile) issue_b(tcol_of(hn, jn), 1 - buf);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int qa = 16 * s + 8 * hi + (gi >> 2);   // rows of the two transposing loads: qa, qa + 4
        v2i p0, p1, s0, s1;
        lds_read_tr4(tr_addr(L::PS, qa), tr_addr(L::PS, qa + 4), tr_addr(L::DS, qa), tr_addr(L::DS, qa + 4), p0, p1,
                     s0, s1);
        const v4i bp = v4i{p0[0], p0[1], p1[0], p1[1]};
        const v4i bs = v4i{s0[0], s0[1], s1[0], s1[1]};
        const int cc = 2 * s + hi;                    // queries 16 s + 8 hi + [0, 8)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int ch = CH * half + 32 * ct + l32;
          const v4i ao = *reinterpret_cast<const v4i*>(sb + L::DOT + ch * 128 + 16 * (cc ^ swz_big(ch, 8)));
          const v4i aq = *reinterpret_cast<const v4i*>(sb + L::QT + ch * 128 + 16 * (cc ^ swz_big(ch, 8)));
          dv[ct] = mfma_bf16(ao, bp, dv[ct]);
          dk[ct] = mfma_bf16(aq, bs, dk[ct]);
        }
      }
    }
    // the scratch and this tile's B buffer are free (group A of tile n + 1 landed before the
    // products); the loads issued above stay in flight.  The accumulators are operands so that
    // the products stay on this side of the barrier (the register allocator otherwise copies
    // them between the two unrolled tiles).
    if constexpr (CT == 2)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : "+v"(dv[0]), "+v"(dv[1]), "+v"(dk[0]), "+v"(dk[CT - 1]) :: "memory");
    else
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : "+v"(dv[0]), "+v"(dk[0]) :: "memory");
    jj = jn;
    hn = h2;
    jn = j2;
  };
  for (int n = 0; n < ntile; n += 2) {
    tile(std::integral_constant<int, 0>{}, n);
    if (n + 1 >= ntile) break;
    tile(std::integral_constant<int, 1>{}, n + 1);
  }

  // ---- store: lane holds key kp + l32, channels CH half + 32 ct + 8 a + 4 hi + [0,4) ----
  const int64_t key = kp + l32;
  uint16_t* dvr = p.dv + (bg * N + key) * D;
  uint16_t* dkr = p.dk + (bg * N + key) * D;
  const float sc = p.scale_nat;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = CH * half + 32 * ct + 8 * a + 4 * hi;
      *reinterpret_cast<uint2*>(dvr + ch) =
          make_uint2(pk_bf16(dv[ct][4 * a], dv[ct][4 * a + 1]), pk_bf16(dv[ct][4 * a + 2], dv[ct][4 * a + 3]));
      *reinterpret_cast<uint2*>(dkr + ch) = make_uint2(pk_bf16(sc * dk[ct][4 * a], sc * dk[ct][4 * a + 1]),
                                                       pk_bf16(sc * dk[ct][4 * a + 2], sc * dk[ct][4 * a + 3]));
    }
}

// ---------------------------------------------------------------------------------------------
// 3b. dK / dV at d = 128 with producer and consumer waves (N % 128 = 0).  A workgroup of eight
// waves owns 128 keys.  In each step waves 0-3 (one per SIMD) run the elementwise phase of query
// tile n while waves 4-7 run the products of tile n - 1, so that every SIMD holds one VALU-heavy
// and one matrix-core-heavy wave at all times; one barrier per step.
//  * elementwise wave e: keys 64 (e / 2) + [0, 64) as two 32-key P blocks, queries 32 (e % 2) +
//    [0, 32).  S^T = K^ Q^T (FP4) and dP^T / l = V^ (dO / l)^T (bf16), one lane per query as in
//    the forward; P~ requantized in registers; dS = p (dP / l - D / l).  P~ (exact in bf16) and
//    dS go to a query-major scratch [64 q][128 keys].
//  * product wave c: keys 64 (c / 2) + [0, 64), channels 64 (c % 2) + [0, 64):
//    dV^T += (dO / l)^T P~ and dK^T += Q^T dS over the tile's 64 queries.  All operands come from
//    row-major tiles through the transposing LDS load (ds_read_b64_tr_b16).
// LDS (163584 bytes): three group-A buffers (Q^ codes and scales, row constants, dO / l; a tile's
// buffer is read by the elementwise phase in one step and by the products in the next), two Q^
// (bf16) buffers and two scratch buffers.  Every LDS access of the two phases is an asm statement
// that waits for its own loads, so buffers are picked at run time without the compiler waiting
// for the direct loads in flight; the barrier of each step waits for everything.
struct DkdvWsLds {
  static constexpr int QC = 0;                  // Q^ codes [64 q][64 B], chunks swizzled (swz_code)
  static constexpr int QS = QC + 4096;          // Q^ scales [64 q] dwords
  static constexpr int ROWS = QS + 256;         // (mq, il, D, D / l) [64 q] float4
  static constexpr int DOS = ROWS + 1024;       // dO / l bf16 [64 q][128], chunks swizzled (x16)
  static constexpr int A_BYTES = DOS + 16384;
  static constexpr int B_BYTES = 16384;         // Q^ bf16 [64 q][128], chunks swizzled (x16)
  static constexpr int S_BYTES = 32768;         // P~ then dS, bf16 [64 q][128 keys] each (x16)
  static constexpr int A0 = 0, B0 = 3 * A_BYTES, S0 = B0 + 2 * B_BYTES;
  static constexpr int BYTES = S0 + 2 * S_BYTES;
};
static_assert(DkdvWsLds::BYTES <= 163840, "LDS");

// 16-byte chunk swizzle of 256-byte rows: a permutation of the 16 chunks within every 16 rows, so
// that 16 consecutive rows read at one logical chunk (the MFMA operand loads), and 4 consecutive
// rows read at two adjacent chunks (the transposing loads, 32 lanes), both spread over all banks.
__device__ __forceinline__ int x16(int q) { return ((q & 3) << 2) | ((q >> 2) & 3); }
__device__ __forceinline__ int x16_off(int q, int c) { return q * 256 + 16 * (c ^ x16(q)); }

template <bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_ws_kernel(BwdParams p) {
  using L = DkdvWsLds;
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int gi = lane & 15, gh = (lane >> 4) & 1;
  const int r4 = wave & 3;
  const int kh = r4 >> 1;                          // 64-key half of the workgroup's keys

  const int64_t N = p.N;
  const int64_t nkt = N / 128;
  const int64_t bg = blockIdx.x / nkt;            // b * Hkv + g
  const int64_t k0 = (blockIdx.x - bg * nkt) * 128;
  const int64_t b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int64_t group = p.Hq / p.Hkv;
  const float c = p.c;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  // ---- staging jobs (one 64-lane LDS-DMA instruction each) ----
  // group A: dO / l (1-KB pieces), Q^ codes (1-KB pieces), Q^ scales, row constants; group B: Q^
  // bf16.  Job j of a group is issued by wave j % 8 in slot j / 8 (the last job repeated where the
  // list runs out).  The query heads of this KV head are contiguous, so one resource per tensor
  // covers them; the tile's first row goes in the scalar offset.
  constexpr int NA = 16 + 4 + 2, NB = 16;
  constexpr int JA = (NA + 7) / 8, JB = NB / 8;
  const int64_t hq0 = b * p.Hq + g * group;       // first query head of this KV head
  const auto qc_rs = make_rsrc(p.q_codes + hq0 * N * (D / 2), group * N * (D / 2));
  const auto qs_rs = make_rsrc(p.q_scales + hq0 * N * (D / 32), group * N * (D / 32));
  const auto rc_rs = make_rsrc(p.rowc + hq0 * N * 4, group * N * 16);
  const auto ds_rs = make_rsrc(p.dos + hq0 * N * D, group * N * D * 2);
  const auto qb_rs = make_rsrc(p.qb + hq0 * N * D, group * N * D * 2);
  // kinds: 0 dO / l, 1 Q^ codes, 2 Q^ scales, 3 row constants | 4 Q^ bf16
  auto kind_a = [](int j) constexpr { return j < 16 ? 0 : j < 20 ? 1 : j == 20 ? 2 : 3; };
  auto goff_of = [&](int kind, int j) -> uint32_t {   // lane's global byte offset within the tile
    if (kind == 0 || kind == 4) {
      const int pos = 64 * j + lane, q = pos >> 4;
      return q * 256 + 16 * ((pos & 15) ^ x16(q));
    }
    if (kind == 1) {
      const int pos = 64 * (j - 16) + lane, q = pos >> 2;
      return q * 64 + 16 * ((pos & 3) ^ swz_code(q, 4));
    }
    return kind == 2 ? 4 * lane : 16 * lane;
  };
  auto dst_of = [](int kind, int j) -> int {
    return kind == 0 ? L::DOS + 1024 * j : kind == 1 ? L::QC + 1024 * (j - 16) : kind == 2 ? L::QS
         : kind == 3 ? L::ROWS : 1024 * j;
  };
  uint32_t goff_a[JA], goff_b[JB];
#pragma unroll
  for (int i = 0; i < JA; ++i) { const int j = min(wave + 8 * i, NA - 1); goff_a[i] = goff_of(kind_a(j), j); }
#pragma unroll
  for (int i = 0; i < JB; ++i) goff_b[i] = goff_of(4, wave + 8 * i);
  auto issue_kind = [&](auto kc, int j, uint32_t goff, int r, int dst_base) __attribute__((always_inline)) {
    constexpr int kind = decltype(kc)::value;
    auto* dst = (__attribute__((address_space(3))) void*)(smem + dst_base + dst_of(kind, j));   // LDS-DMA target
    if constexpr (kind == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(ds_rs, dst, 16, (int)goff, r * (D * 2), 0, 0);
    else if constexpr (kind == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(qc_rs, dst, 16, (int)goff, r * (D / 2), 0, 0);
    else if constexpr (kind == 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(qs_rs, dst, 4, (int)goff, r * (D / 32), 0, 0);
    else if constexpr (kind == 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(rc_rs, dst, 16, (int)goff, r * 16, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(qb_rs, dst, 16, (int)goff, r * (D * 2), 0, 0);
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;
  using K4 = std::integral_constant<int, 4>;
  // group A of the tile whose first row is r into A buffer a; group B into B buffer bq
  auto issue_a = [&](int r, int a) __attribute__((always_inline)) {
    const int base = L::A0 + a * L::A_BYTES;
    issue_kind(K0{}, wave, goff_a[0], r, base);
    issue_kind(K0{}, wave + 8, goff_a[1], r, base);
    const int j = min(wave + 16, NA - 1);
    if (j < 20) issue_kind(K1{}, j, goff_a[2], r, base);
    else if (j == 20) issue_kind(K2{}, j, goff_a[2], r, base);
    else issue_kind(K3{}, j, goff_a[2], r, base);
  };
  auto issue_b = [&](int r, int bq) __attribute__((always_inline)) {
    const int base = L::B0 + bq * L::B_BYTES;
    issue_kind(K4{}, wave, goff_b[0], r, base);
    issue_kind(K4{}, wave + 8, goff_b[1], r, base);
  };
  static_assert(JA == 3 && JB == 2, "job slots");

  // ---- query tiles: the query heads of the group, and per head the tiles that see any key ----
  // (wave-uniform 32-bit scalars: group * D * N * 2 < 2^31 is checked at the boundary)
  const int j_first = CAUSAL ? (int)(k0 / 64) : 0;
  const int nj = (int)(N / 64) - j_first;
  const int ntile = (int)group * nj;
  auto row_of = [&](int h_, int j_) __attribute__((always_inline)) {   // first row of [head][N]
    return __builtin_amdgcn_readfirstlane(h_ * (int)N + (j_first + j_) * 64);
  };
  auto next = [&](int& h_, int& j_) __attribute__((always_inline)) {
    if (++j_ == nj) { j_ = 0; ++h_; }
  };
  // Step m (0 .. ntile) issues group A of tile m + 1 and group B of tile m; the elementwise waves
  // take tile m, the product waves tile m - 1.  Buffers rotate: A over three (tile n in n % 3), B
  // and the scratch over two (n % 2).
  int hA = 0, jA = 0;                              // tile m + 1
  next(hA, jA);
  int hB = 0, jB = 0;                              // tile m
  int am = 0;                                      // m % 3
  auto step_loads = [&](int m) __attribute__((always_inline)) {
    if (m + 1 < ntile) issue_a(row_of(hA, jA), am == 2 ? 0 : am + 1);
    if (m < ntile) issue_b(row_of(hB, jB), m & 1);
  };
  auto step_end = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    hB = hA;
    jB = jA;
    next(hA, jA);
    am = am == 2 ? 0 : am + 1;
  };
  issue_a(row_of(0, 0), 0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  if (wave < 4) {
    // ================= elementwise waves =================
    const int qh = r4 & 1;
    const int ql = 32 * qh + l32;                  // this lane's query within the tile
    // constant operands: K^ (FP4) and V^ (bf16) rows of the wave's two 32-key blocks, in the row
    // order that makes lane l hold keys kp + 16 (l / 32) + r in S^T / dP^T register r
    v4i ka[2][2], va[2][8];
    int ksc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int64_t krow = k0 + 64 * kh + 32 * kt + row_key(l32);
      const uint8_t* kr = p.k_codes + (bg * N + krow) * (D / 2);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ka[kt][ks] = *reinterpret_cast<const v4i*>(kr + 16 * hi + 32 * ks);
      const uint8_t* ksr = p.k_scales + (bg * N + krow) * (D / 32);
      ksc[kt] = (int)(ksr[hi] | (ksr[2 + hi] << 16));
      const uint16_t* vr = p.vb + (bg * N + krow) * D;
#pragma unroll
      for (int s = 0; s < 8; ++s) va[kt][s] = *reinterpret_cast<const v4i*>(vr + 16 * s + 8 * hi);
    }
    // per-lane LDS offsets within a group-A buffer and within a scratch buffer
    const uint32_t o_qc0 = L::QC + ql * 64 + 16 * (hi ^ swz_code(ql, 4));
    const uint32_t o_qc1 = L::QC + ql * 64 + 16 * ((hi + 2) ^ swz_code(ql, 4));
    const uint32_t o_qs = L::QS + 4 * ql, o_rc = L::ROWS + 16 * ql;
    uint32_t o_do[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) o_do[s] = L::DOS + x16_off(ql, 2 * s + hi);
    // scratch: row ql, keys 64 kh + 32 kt + 16 hi + [0, 16) = chunks 8 kh + 4 kt + 2 hi + {0, 1}
    uint32_t o_sc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) o_sc[kt][u] = x16_off(ql, 8 * kh + 4 * kt + 2 * hi + u);

    for (int m = 0; m <= ntile; ++m) {
      step_loads(m);
      if (m < ntile) {
        const uint32_t ab = lds0 + L::A0 + am * L::A_BYTES;
        const uint32_t sb = lds0 + L::S0 + (m & 1) * L::S_BYTES;
        v4i q0v, q1v, rcv, dov[8];
        uint32_t qsw;
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %13\n\t"
            "ds_read_b32 %2, %14\n\t"
            "ds_read_b128 %3, %15\n\t"
            "ds_read_b128 %4, %16\n\t"
            "ds_read_b128 %5, %17\n\t"
            "ds_read_b128 %6, %18\n\t"
            "ds_read_b128 %7, %19\n\t"
            "ds_read_b128 %8, %20\n\t"
            "ds_read_b128 %9, %21\n\t"
            "ds_read_b128 %10, %22\n\t"
            "ds_read_b128 %11, %23\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(q0v), "=&v"(q1v), "=&v"(qsw), "=&v"(rcv), "=&v"(dov[0]), "=&v"(dov[1]), "=&v"(dov[2]),
              "=&v"(dov[3]), "=&v"(dov[4]), "=&v"(dov[5]), "=&v"(dov[6]), "=&v"(dov[7])
            : "v"(ab + o_qc0), "v"(ab + o_qc1), "v"(ab + o_qs), "v"(ab + o_rc), "v"(ab + o_do[0]), "v"(ab + o_do[1]),
              "v"(ab + o_do[2]), "v"(ab + o_do[3]), "v"(ab + o_do[4]), "v"(ab + o_do[5]), "v"(ab + o_do[6]),
              "v"(ab + o_do[7]));
        const int qsc = (int)(qsw >> (8 * hi));
        const float mq = __int_as_float(rcv[0]), ddl = __int_as_float(rcv[3]);
        const int qrow = (j_first + jB) * 64 + ql;  // query position (causal mask)
        v4i outp[2][2], outs[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          v16f st = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka[kt][0]), widen(q0v), v16f{}, 4, 4, 0,
                                                                   ksc[kt], 0, qsc);
          st = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka[kt][1]), widen(q1v), st, 4, 4, 2, ksc[kt], 2,
                                                               qsc);
          // dP^T - D/l: the accumulator starts at -D/l, so dS needs one multiply per element
          v16f dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = -ddl;
#pragma unroll
          for (int s = 0; s < 8; ++s) dp = mfma_bf16(va[kt][s], dov[s], dp);
          // register r holds key kp + 16 hi + r
          if (CAUSAL) {
            const int jrel = qrow - (int)(k0 + 64 * kh + 32 * kt) - 16 * hi;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (r > jrel) st[r] = -__builtin_inff();
          }
          float mx = st[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
          auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          const float bmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          const int sbyte = p_scale_byte(__builtin_fmaf(bmax, c, -mq), mq);
          const float sc = __uint_as_float((uint32_t)sbyte << 23);
          float pr[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c, -mq));
          uint32_t aw[8], sw8[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t u = 0;
            u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, pr[4 * q], pr[4 * q + 1], sc, 0);
            u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, pr[4 * q + 2], pr[4 * q + 3], sc, 1);
            aw[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, sc, 0));
            aw[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, sc, 1));
            sw8[2 * q] = pk_bf16(pr[4 * q] * dp[4 * q], pr[4 * q + 1] * dp[4 * q + 1]);
            sw8[2 * q + 1] = pk_bf16(pr[4 * q + 2] * dp[4 * q + 2], pr[4 * q + 3] * dp[4 * q + 3]);
          }
          outp[kt][0] = v4i{(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3]};
          outp[kt][1] = v4i{(int)aw[4], (int)aw[5], (int)aw[6], (int)aw[7]};
          outs[kt][0] = v4i{(int)sw8[0], (int)sw8[1], (int)sw8[2], (int)sw8[3]};
          outs[kt][1] = v4i{(int)sw8[4], (int)sw8[5], (int)sw8[6], (int)sw8[7]};
        }
        // P~ at +0, dS at +16384 of the scratch buffer (the trailing nop covers the store-data
        // hazard of the last 128-bit store)
        asm volatile(
            "ds_write_b128 %0, %4\n\t"
            "ds_write_b128 %1, %5\n\t"
            "ds_write_b128 %2, %6\n\t"
            "ds_write_b128 %3, %7\n\t"
            "ds_write_b128 %0, %8 offset:16384\n\t"
            "ds_write_b128 %1, %9 offset:16384\n\t"
            "ds_write_b128 %2, %10 offset:16384\n\t"
            "ds_write_b128 %3, %11 offset:16384\n\t"
            "s_nop 1"
            :
            : "v"(sb + o_sc[0][0]), "v"(sb + o_sc[0][1]), "v"(sb + o_sc[1][0]), "v"(sb + o_sc[1][1]),
              "v"(outp[0][0]), "v"(outp[0][1]), "v"(outp[1][0]), "v"(outp[1][1]), "v"(outs[0][0]), "v"(outs[0][1]),
              "v"(outs[1][0]), "v"(outs[1][1])
            : "memory");
      }
      step_end();
    }
  } else {
    // ================= product waves =================
    const int chh = r4 & 1;                        // 64-channel half
    v16f dv[2][2], dk[2][2];                       // [key block kt][channel tile ct]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        dv[kt][ct] = v16f{};
        dk[kt][ct] = v16f{};
      }
    // transposing loads.  In each 16-lane group, lane i supplies four consecutive elements of row
    // base + i / 4 and lane j receives element j of rows base .. base + 3.
    //  * scratch (B operands): keys 64 kh + 32 kt + 16 gh + 4 (gi % 4) of rows 16 s + 8 hi + gi / 4
    //    and + 4: lane l receives key 64 kh + 32 kt + l % 32 of queries 16 s + 8 hi + [0, 8);
    //  * dO / l and Q^ (A operands): channels 64 chh + 32 ct + 16 gh + 4 (gi % 4) of the same rows:
    //    lane l receives channel 64 chh + 32 ct + l % 32 of those queries.
    // The swizzle is periodic in 16 rows, so step s (rows + 16 s) is an immediate offset of 4096 s.
    const int qa = 8 * hi + (gi >> 2);
    uint32_t o_p[2][2], o_a[2][2];                 // [kt or ct][u: rows qa or qa + 4]
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = 64 * kh + 32 * t + 16 * gh + 4 * (gi & 3);
        o_p[t][u] = x16_off(qa + 4 * u, key >> 3) + 2 * (key & 7);
        const int ch = 64 * chh + 32 * t + 16 * gh + 4 * (gi & 3);
        o_a[t][u] = x16_off(qa + 4 * u, ch >> 3) + 2 * (ch & 7);
      }
    for (int m = 0; m <= ntile; ++m) {
      step_loads(m);
      if (m >= 1) {
        const int n = m - 1;                       // the tile of these products (A buffer n % 3)
        const uint32_t ab = lds0 + L::A0 + (am == 0 ? 2 : am - 1) * L::A_BYTES + L::DOS;
        const uint32_t bb = lds0 + L::B0 + (n & 1) * L::B_BYTES;
        const uint32_t sb = lds0 + L::S0 + (n & 1) * L::S_BYTES;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v2i rp[2][2], rs[2][2], ro[2][2], rq[2][2];
          asm volatile(
              "ds_read_b64_tr_b16 %0, %16 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %1, %17 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %2, %18 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %3, %19 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %4, %16 offset:%c29\n\t"
              "ds_read_b64_tr_b16 %5, %17 offset:%c29\n\t"
              "ds_read_b64_tr_b16 %6, %18 offset:%c29\n\t"
              "ds_read_b64_tr_b16 %7, %19 offset:%c29\n\t"
              "ds_read_b64_tr_b16 %8, %20 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %9, %21 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %10, %22 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %11, %23 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %12, %24 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %13, %25 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %14, %26 offset:%c28\n\t"
              "ds_read_b64_tr_b16 %15, %27 offset:%c28\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(rp[0][0]), "=&v"(rp[0][1]), "=&v"(rp[1][0]), "=&v"(rp[1][1]), "=&v"(rs[0][0]), "=&v"(rs[0][1]),
                "=&v"(rs[1][0]), "=&v"(rs[1][1]), "=&v"(ro[0][0]), "=&v"(ro[0][1]), "=&v"(ro[1][0]), "=&v"(ro[1][1]),
                "=&v"(rq[0][0]), "=&v"(rq[0][1]), "=&v"(rq[1][0]), "=&v"(rq[1][1])
              : "v"(sb + o_p[0][0]), "v"(sb + o_p[0][1]), "v"(sb + o_p[1][0]), "v"(sb + o_p[1][1]),
                "v"(ab + o_a[0][0]), "v"(ab + o_a[0][1]), "v"(ab + o_a[1][0]), "v"(ab + o_a[1][1]),
                "v"(bb + o_a[0][0]), "v"(bb + o_a[0][1]), "v"(bb + o_a[1][0]), "v"(bb + o_a[1][1]),
                "n"(4096 * s), "n"(4096 * s + 16384));
          v4i bp[2], bs[2], ao[2], aq[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            bp[t] = v4i{rp[t][0][0], rp[t][0][1], rp[t][1][0], rp[t][1][1]};
            bs[t] = v4i{rs[t][0][0], rs[t][0][1], rs[t][1][0], rs[t][1][1]};
            ao[t] = v4i{ro[t][0][0], ro[t][0][1], ro[t][1][0], ro[t][1][1]};
            aq[t] = v4i{rq[t][0][0], rq[t][0][1], rq[t][1][0], rq[t][1][1]};
          }
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              dv[kt][ct] = mfma_bf16(ao[ct], bp[kt], dv[kt][ct]);
              dk[kt][ct] = mfma_bf16(aq[ct], bs[kt], dk[kt][ct]);
            }
        }
      }
      step_end();
    }
    // ---- store: lane holds key k0 + 64 kh + 32 kt + l32, channels 64 chh + 32 ct + 8 a + 4 hi + [0, 4) ----
    const float sc = p.scale_nat;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int64_t key = k0 + 64 * kh + 32 * kt + l32;
      uint16_t* dvr = p.dv + (bg * N + key) * D;
      uint16_t* dkr = p.dk + (bg * N + key) * D;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int ch = 64 * chh + 32 * ct + 8 * a4 + 4 * hi;
          *reinterpret_cast<uint2*>(dvr + ch) = make_uint2(pk_bf16(dv[kt][ct][4 * a4], dv[kt][ct][4 * a4 + 1]),
                                                           pk_bf16(dv[kt][ct][4 * a4 + 2], dv[kt][ct][4 * a4 + 3]));
          *reinterpret_cast<uint2*>(dkr + ch) =
              make_uint2(pk_bf16(sc * dk[kt][ct][4 * a4], sc * dk[kt][ct][4 * a4 + 1]),
                         pk_bf16(sc * dk[kt][ct][4 * a4 + 2], sc * dk[kt][ct][4 * a4 + 3]));
        }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 4. dQ.  Workgroup = W waves of 32 query rows; key tiles of 64 staged in LDS: a step computes GT
// tiles from one half of the stages while the other half is refilled with the next GT tiles.
template <int D>
struct DqLds {
  static constexpr int KC = 0;                        // K^ codes [64 slots][D/2], as in the forward
  static constexpr int KS = KC + 64 * D / 2;          // K^ scales [64 slots] dwords
  static constexpr int VB = KS + 64 * 4;              // V^ bf16 [64 slots][D], swizzled chunks
  static constexpr int KT = VB + 64 * D * 2;          // K^T bf16 [D][64 keys], swizzled chunks
  static constexpr int BYTES = KT + D * 64 * 2;
};

template <int D, int W, bool CAUSAL>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdParams p) {
  using L = DqLds<D>;
  constexpr int NT = 64 * W;
  constexpr int KS_STEPS = D / 64;
  constexpr int DS_STEPS = D / 16;
  constexpr int CT = D / 32;
  constexpr int KCH = D / 32;             // 16-B chunks per K^ code row
  // key tiles per barrier: two (four stages) when that fits the LDS of every workgroup the two
  // waves per SIMD allow on a CU, else one (two stages).  Measured at the QAT shape (eight-wave
  // workgroups, one per CU): backward 1.3546-1.3549 against 1.3644-1.3657 ms, outputs identical.
  constexpr int GT = (8 / W) * 2 * 2 * L::BYTES <= 160 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * GT * L::BYTES];   // two halves of GT stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int64_t N = p.N;
  const int64_t nqt = N / (32 * W);
  const int64_t bh = blockIdx.x / nqt;
  int64_t qt = blockIdx.x - bh * nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int64_t b = bh / p.Hq, h = bh - b * p.Hq;
  const int64_t g = h / (p.Hq / p.Hkv);
  const int64_t bg = b * p.Hkv + g;
  const int64_t q0 = qt * 32 * W;
  const int64_t qw = q0 + 32 * wave;
  const int64_t row = qw + l32;
  const float c = p.c;

  // the wave's Q^ (FP4 B operand of S^T) and dO (bf16 B operand of dP^T), fixed for the kernel
  v4i qb[KS_STEPS];
  int qsc;
  {
    const uint8_t* qr = p.q_codes + (bh * N + row) * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS_STEPS; ++ks) qb[ks] = *reinterpret_cast<const v4i*>(qr + 16 * hi + 32 * ks);
    const uint8_t* qs = p.q_scales + (bh * N + row) * (D / 32);
    qsc = (D == 128) ? (int)(qs[hi] | (qs[2 + hi] << 16)) : (int)qs[hi];
  }
  v4i ob[DS_STEPS];
  {
    const uint16_t* orow = p.dout + (bh * N + row) * D;
#pragma unroll
    for (int s = 0; s < DS_STEPS; ++s) ob[s] = *reinterpret_cast<const v4i*>(orow + 16 * s + 8 * hi);
  }
  const float4 rc = reinterpret_cast<const float4*>(p.rowc)[bh * N + row];
  const float mq = rc.x, il = rc.y, dd = rc.z;

  v16f acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v16f{};

  const int ntiles = (int)(CAUSAL ? ((q0 + 32 * W - 1) / 64 + 1) : (N / 64));
  const int last_active = CAUSAL ? (int)((qw + 31) / 64) : ntiles - 1;

  // ---- key-tile staging: direct global -> LDS loads into two stages, one tile ahead ----
  // Jobs (one 64-lane LDS-DMA instruction each): K^ codes, V^ bf16 and K^T bf16 in 1-KB pieces,
  // then the K^ scales (one dword per slot).  The LDS layouts (slot permutation, chunk swizzles)
  // come from each lane's global source.  Wave w issues jobs w, w + W, ...; each wave issues JPW
  // per tile, the last job repeated where the list runs out (an identical rewrite).
  constexpr int VC = D / 8;               // 16-B chunks per V^ bf16 row
  constexpr int NKC = 64 * D / 2 / 1024, NVB = 64 * D * 2 / 1024, NKT = D * 64 * 2 / 1024;
  constexpr int NJ = NKC + NVB + NKT + 1;
  constexpr int JPW = (NJ + W - 1) / W;
  const auto kc_rs = make_rsrc(p.k_codes + bg * N * (D / 2), N * (D / 2));
  const auto ks_rs = make_rsrc(p.k_scales + bg * N * (D / 32), N * (D / 32));
  const auto vb_rs = make_rsrc(p.vb + bg * N * D, N * D * 2);
  const auto kt_rs = make_rsrc(p.kt + bg * D * N, N * D * 2);
  auto kind_of = [](int j) constexpr { return j < NKC ? 0 : j < NKC + NVB ? 1 : j < NKC + NVB + NKT ? 2 : 3; };
  // lane's global byte offset (within tile 0) and LDS destination of job j
  auto job_goff_of = [&](int j) -> uint32_t {
    if (j < NKC) {
      const int cidx = 64 * j + lane, s = cidx / KCH, cc = (cidx % KCH) ^ swz_code(s, KCH);
      return (32 * (s >> 5) + row_key(s & 31)) * (D / 2) + 16 * cc;
    } else if (j < NKC + NVB) {
      const int cidx = 64 * (j - NKC) + lane, s = cidx / VC, cc = (cidx % VC) ^ swz_big(s, VC);
      return (32 * (s >> 5) + row_key(s & 31)) * (D * 2) + 16 * cc;
    } else if (j < NKC + NVB + NKT) {
      const int cidx = 64 * (j - NKC - NVB) + lane, ch = cidx >> 3, cc = (cidx & 7) ^ swz_big(ch, 8);
      return (uint32_t)ch * (uint32_t)(N * 2) + 16 * cc;
    }
    return (32 * (lane >> 5) + row_key(lane & 31)) * (D / 32);
  };
  auto job_dst_of = [](int j) -> int {
    return j < NKC ? L::KC + 1024 * j
         : j < NKC + NVB ? L::VB + 1024 * (j - NKC)
         : j < NKC + NVB + NKT ? L::KT + 1024 * (j - NKC - NVB) : L::KS;
  };
  // with few jobs per wave the lane offsets are kept in registers, else recomputed per tile
  constexpr bool PRE = JPW <= 6;
  uint32_t job_goff[PRE ? JPW : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < JPW; ++i) job_goff[i] = job_goff_of(min(wave + W * i, NJ - 1));
  }
  auto issue_kind = [&](int kind, int i, int t, uint8_t* stage) __attribute__((always_inline)) {
    const int j = min(wave + W * i, NJ - 1);
    auto* dst = (__attribute__((address_space(3))) void*)(stage + job_dst_of(j));   // LDS-DMA target
    uint32_t goff;
    if constexpr (PRE) goff = job_goff[PRE ? i : 0];
    else goff = job_goff_of(j);
    if (kind == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kc_rs, dst, 16, (int)goff, t * (64 * D / 2), 0, 0);
    } else if (kind == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vb_rs, dst, 16, (int)goff, t * (64 * D * 2), 0, 0);
    } else if (kind == 2) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kt_rs, dst, 16, (int)goff, t * (64 * 2), 0, 0);
    } else {                                  // d/32 scale bytes per slot, one dword per lane
      if constexpr (D == 128) __builtin_amdgcn_raw_ptr_buffer_load_lds(ks_rs, dst, 4, (int)goff, t * (64 * D / 32), 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(ks_rs, dst, 2, (int)goff, t * (64 * D / 32), 0, 0);
    }
  };
  auto issue_job = [&](auto ic, int t, uint8_t* stage) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < JPW) {
      constexpr int klo = kind_of(W * i < NJ - 1 ? W * i : NJ - 1);
      constexpr int khi = kind_of(W * i + W - 1 < NJ - 1 ? W * i + W - 1 : NJ - 1);
      if constexpr (klo == khi) issue_kind(klo, i, t, stage);
      else issue_kind(kind_of(min(wave + W * i, NJ - 1)), i, t, stage);
    }
  };
  auto issue_tile = [&](int t, uint8_t* stage) __attribute__((always_inline)) {
    t = __builtin_amdgcn_readfirstlane(t);
    static_assert(JPW <= 20, "job slots");
    issue_job(std::integral_constant<int, 0>{}, t, stage);
    issue_job(std::integral_constant<int, 1>{}, t, stage);
    issue_job(std::integral_constant<int, 2>{}, t, stage);
    issue_job(std::integral_constant<int, 3>{}, t, stage);
    issue_job(std::integral_constant<int, 4>{}, t, stage);
    issue_job(std::integral_constant<int, 5>{}, t, stage);
    issue_job(std::integral_constant<int, 6>{}, t, stage);
    issue_job(std::integral_constant<int, 7>{}, t, stage);
    issue_job(std::integral_constant<int, 8>{}, t, stage);
    issue_job(std::integral_constant<int, 9>{}, t, stage);
    issue_job(std::integral_constant<int, 10>{}, t, stage);
    issue_job(std::integral_constant<int, 11>{}, t, stage);
    issue_job(std::integral_constant<int, 12>{}, t, stage);
    issue_job(std::integral_constant<int, 13>{}, t, stage);
    issue_job(std::integral_constant<int, 14>{}, t, stage);
    issue_job(std::integral_constant<int, 15>{}, t, stage);
    issue_job(std::integral_constant<int, 16>{}, t, stage);
    issue_job(std::integral_constant<int, 17>{}, t, stage);
    issue_job(std::integral_constant<int, 18>{}, t, stage);
    issue_job(std::integral_constant<int, 19>{}, t, stage);
  };

  auto compute = [&](int t, const uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int slot = 32 * T + l32;
      // S^T (FP4) for the 32 keys of half T
      const uint32_t kw = *reinterpret_cast<const uint32_t*>(base + L::KS + 4 * slot);
      const int ksc = (int)(kw >> (8 * hi));
      v16f st = v16f{};
#pragma unroll
      for (int ks = 0; ks < KS_STEPS; ++ks) {
        const int pc = (hi + 2 * ks) ^ swz_code(slot, KCH);
        const v4i ka = *reinterpret_cast<const v4i*>(base + L::KC + slot * (D / 2) + 16 * pc);
        if (ks == 0)
          st = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka), widen(qb[0]), st, 4, 4, 0, ksc, 0, qsc);
        else
          st = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka), widen(qb[KS_STEPS - 1]), st, 4, 4, 2, ksc,
                                                              2, qsc);
      }
      // dP^T = V^ dO^T (bf16)
      v16f dp = v16f{};
#pragma unroll
      for (int s = 0; s < DS_STEPS; ++s) {
        const int cc = 2 * s + hi;
        const v4i a = *reinterpret_cast<const v4i*>(base + L::VB + slot * 2 * D + 16 * (cc ^ swz_big(slot, D / 8)));
        dp = mfma_bf16(a, ob[s], dp);
      }
      // dS l = p (dP - D), p = exp2(s c - m log2 e): the row's 1/l is applied to the finished dQ
      // row instead of to every pair; register r holds key 64t + 32T + 16hi + r
      if (CAUSAL && ((int64_t)t * 64 + 63 > qw)) {
        const int jrel = (int)(row - (int64_t)t * 64) - 32 * T - 16 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r > jrel) st[r] = -__builtin_inff();
      }
      uint32_t dsw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * i], c, -mq));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * i + 1], c, -mq));
        dsw[i] = pk_bf16(p0 * (dp[2 * i] - dd), p1 * (dp[2 * i + 1] - dd));
      }
      // dQ^T += K^T dS^T: k-step s2 takes keys 32T + 16 hi + 8 s2 + [0, 8) (registers 8 s2..)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const v4i bsv = v4i{(int)dsw[4 * s2], (int)dsw[4 * s2 + 1], (int)dsw[4 * s2 + 2], (int)dsw[4 * s2 + 3]};
        const int cc = 4 * T + 2 * hi + s2;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int ch = 32 * ct + l32;
          const v4i a = *reinterpret_cast<const v4i*>(base + L::KT + ch * 128 + 16 * (cc ^ swz_big(ch, 8)));
          acc[ct] = mfma_bf16(a, bsv, acc[ct]);
        }
      }
    }
  };

  // step at tile t: refill the other half of the stages (freed by the barrier that ended the
  // previous step) with tiles t + GT .. t + 2 GT - 1, then compute tiles t .. t + GT - 1; the
  // barrier that ends the step publishes the refilled half (each wave first waits for its own DMAs
  // and LDS reads) and frees the half just computed.  The asm statements also keep the compiler
  // from moving memory accesses across the barrier.
  for (int k = 0; k < GT; ++k)
    if (k < ntiles) issue_tile(k, smem + k * L::BYTES);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  auto step = [&](int t, auto hc) __attribute__((always_inline)) {
    constexpr int s0 = decltype(hc)::value ? GT : 0, l0 = GT - s0;
#pragma unroll
    for (int i = 0; i < GT; ++i)
      if (t + GT + i < ntiles) issue_tile(t + GT + i, smem + (l0 + i) * L::BYTES);
#pragma unroll
    for (int i = 0; i < GT; ++i)
      if (t + i < ntiles && t + i <= last_active) compute(t + i, smem + (s0 + i) * L::BYTES);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  for (int t = 0; t < ntiles; t += 2 * GT) {
    step(t, std::integral_constant<int, 0>{});
    if (t + GT >= ntiles) break;
    step(t + GT, std::integral_constant<int, 1>{});
  }

  // ---- store dQ = scale / l * dQ^T: lane holds query `row`, channels 32 ct + 8 a + 4 hi + [0,4) ----
  uint16_t* dqr = p.dq + (bh * N + row) * D;
  const float sc = p.scale_nat * il;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * ct + 8 * a + 4 * hi;
      *reinterpret_cast<uint2*>(dqr + ch) = make_uint2(pk_bf16(sc * acc[ct][4 * a], sc * acc[ct][4 * a + 1]),
                                                       pk_bf16(sc * acc[ct][4 * a + 2], sc * acc[ct][4 * a + 3]));
    }
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

template <int D, bool CAUSAL>
hipError_t launch_main(const BwdParams& p, hipStream_t stream) {
  if (D == 128 && p.N % 128 == 0)
    hipLaunchKernelGGL((bwd_dkdv_ws_kernel<CAUSAL>), dim3((unsigned)((p.N / 128) * p.Hkv * p.B)), dim3(512), 0,
                       stream, p);
  else if (p.N % 128 == 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 8, CAUSAL>), dim3((unsigned)((p.N / 128) * p.Hkv * p.B)), dim3(512), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 4, CAUSAL>), dim3((unsigned)((p.N / 64) * p.Hkv * p.B)), dim3(256), 0,
                       stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.N % 256 == 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, 8, CAUSAL>), dim3((unsigned)((p.N / 256) * p.Hq * p.B)), dim3(512), 0,
                       stream, p);
  } else if (p.N % 128 == 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, 4, CAUSAL>), dim3((unsigned)((p.N / 128) * p.Hq * p.B)), dim3(256), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<D, 2, CAUSAL>), dim3((unsigned)((p.N / 64) * p.Hq * p.B)), dim3(128), 0,
                       stream, p);
  }
  return hipGetLastError();
}

}  // namespace

BwdWorkspace bwd_workspace_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
  BwdWorkspace w;
  w.rowc = 0;
  w.vb = w.rowc + align256(B * Hq * N * 16);
  w.kt = w.vb + align256(B * Hkv * N * d * 2);
  w.qt = w.kt + align256(B * Hkv * N * d * 2);
  w.dot = w.qt + align256(B * Hq * N * d * 2);
  w.total = w.dot + align256(B * Hq * N * d * 2);
  return w;
}

hipError_t launch_bwd(const BwdParams& p0, hipStream_t stream) {
  // d = 128 with N % 128 = 0 runs the producer/consumer dK/dV kernel, which reads row-major
  // Q^ (bf16) and dO / l written by the row pass into the regions of the transposed copies
  const bool ws = p0.d == 128 && p0.N % 128 == 0;
  BwdParams p = p0;
  p.qb = ws ? p.qt : nullptr;
  p.dos = ws ? p.dot : nullptr;
  const int64_t rows = p.B * p.Hq * p.N;
  hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p.o, p.dout, p.m,
                     p.l, p.rowc, rows, (int)p.d, p.q_codes, p.q_scales, p.qb, p.dos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t d = p.d, N = p.N;
  // V^ codes (block-major [N/32][d][16]) -> V^ bf16 [N][d]
  hipLaunchKernelGGL((bwd_transpose_kernel<true, true>), dim3((unsigned)(N / 64), (unsigned)(d / 64), (unsigned)(p.B * p.Hkv)),
                     dim3(256), 0, stream, p.v_codes, p.v_scales, p.vb, d, N);
  // K^ codes [N][d/2] -> K^T bf16 [d][N] (dQ); for the other dK/dV kernel also Q^ likewise and
  // dO bf16 [N][d] -> dO^T [d][N], carrying each query's 1/l: dV^T = dO^T diag(1/l) P~
  hipLaunchKernelGGL(bwd_transpose_kernel<true>, dim3((unsigned)(d / 64), (unsigned)(N / 64), (unsigned)(p.B * p.Hkv)),
                     dim3(256), 0, stream, p.k_codes, p.k_scales, p.kt, N, d);
  if (!ws) {
    hipLaunchKernelGGL(bwd_transpose_kernel<true>, dim3((unsigned)(d / 64), (unsigned)(N / 64), (unsigned)(p.B * p.Hq)),
                       dim3(256), 0, stream, p.q_codes, p.q_scales, p.qt, N, d);
    hipLaunchKernelGGL(bwd_transpose_kernel<false>, dim3((unsigned)(d / 64), (unsigned)(N / 64), (unsigned)(p.B * p.Hq)),
                       dim3(256), 0, stream, (const uint8_t*)p.dout, (const uint8_t*)nullptr, p.dot, N, d,
                       (const float*)p.rowc + 1);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.d == 128) return p.causal ? launch_main<128, true>(p, stream) : launch_main<128, false>(p, stream);
  return p.causal ? launch_main<64, true>(p, stream) : launch_main<64, false>(p, stream);
}

}  // namespace attnfp4
