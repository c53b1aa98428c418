// MXFP4 FlashAttention-style forward kernel for gfx950.
//
// The computation (Attn-QAT abstract: FP4 attention forward; HiFA4 abstract: QK^T and PV as
// 4-bit GEMMs with a wider online-softmax state; EFQ-Softmax abstract: exp-then-quantize P, the
// same quantized P in the PV numerator and the P.1 denominator, FlashAttention's running max,
// history rescaling, wide accumulation and final normalisation):
//   per query row, over ascending 64-key tiles:
//     s = q^.k^ (raw, fp32 from the scaled FP4 MFMA),  m' = max(m, max s)
//     p = exp(scale * (s - m')),  P~ = MXFP4(p) per 32-key block
//     l = alpha l + sum P~,  acc = alpha acc + P~ V^,  alpha = exp(scale * (m - m'))
//   O = acc / l (bf16), saved m (natural-log units) and l.
//
// gfx950 mapping.  One wave owns 32 query rows; a workgroup of W waves shares each 64-key
// K^/V^ tile through LDS (stages filled by direct global-to-LDS loads: three tiles computed per
// barrier from one half of six stages while the other half is refilled, see tiles_per_step).  On
// gfx950 the matrix core and the vector ALU barely overlap, so a tile
// costs about the sum of its MFMA time and its VALU time (exp, E2M1 conversion, max, FMA); the
// kernel is shaped for three waves per SIMD, which measured best, and keeps everything else (tile
// loads, LDS reads, barriers) under that sum.
//
// The same kernel serves the cache forward (KV: new rows against a quantized key/value cache,
// bottom-right causal, per-sequence lengths, query heads of a GQA group packed into the waves) and
// the middle pass of its split form (SPLIT: one range of key tiles per workgroup).  The split form's
// other passes are in fwd_split.hip: kv_max_kernel (each range's largest visible score) and
// kv_merge_kernel (the ranges' partial results into O, m, l).  The kernel template is shared by
// fwd.hip (plain and one-pass cache launches) and fwd_split.hip, which are compiled with different
// scheduler settings.
//  * S is computed transposed, S^T = K^ Q^T, with V_MFMA_SCALE_F32_32X32X64_F8F6F4 (A = K^ rows
//    from LDS, B = the wave's Q^ held in registers for the whole kernel).  The 64 K^ rows of a
//    tile are staged with a permutation of the keys (slot_key) chosen so that, in the output
//    layout of the two S^T MFMAs, lane l holds all 32 keys of P block l/32 for query l%32 (key
//    32(l/32) + 16T + r in register r of MFMA T).
//  * Each lane therefore finds its block maximum alone; one permlane32 swap with the partner lane
//    gives the tile maximum.  The lane converts its 32 values with the hardware E2M1 conversion
//    (v_cvt_scalef32_pk_fp4_f32) against its block's E8M0 scale, and the packed codes are in
//    the B-operand layout of the scaled FP4 MFMA as they stand, with that scale as the lane's B
//    scale.
//  * O is accumulated transposed, O^T = V^T P~^T (A = the V^ tile as [d][64 keys] in LDS, staged
//    from the block-major V^ layout; B = the packed P~), so each lane's accumulators belong to
//    one query and the history
//    rescale needs no cross-lane traffic; it is skipped when no row of the wave raised its max.
//  * The denominator sum of P~ runs on the matrix core too: one 16x16x128 scaled MFMA with a
//    constant 0/1 A operand reduces the same packed P~ registers to per-query row sums.
#pragma once

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace attnfp4 {

namespace {

constexpr int BC = 64;  // key-tile width; part of the definition of P quantization
constexpr int64_t kCuPerXcd = 32;   // MI355X: 256 compute units in 8 XCDs

template <int D>
struct Stage {
  static constexpr int KC_BYTES = BC * D / 2;   // K^ codes, [slot][d/2], swizzled 16-B chunks
  // (the LDS-DMA loads of 1 and 2 bytes write one zero-extended dword per lane)
  static constexpr int KS_BYTES = BC * 4;       // K^ scales, [slot][4]: d/32 blocks, zero padded
  static constexpr int VC_BYTES = D * BC / 2;   // V^ codes, [d][64 keys / 2], swizzled chunks
  static constexpr int VS_BYTES = 256;          // V^ scales as in memory: [2 blocks][d] (d = 64: half used)
  static constexpr int KC = 0;
  static constexpr int KS = KC + KC_BYTES;
  static constexpr int VC = KS + KS_BYTES;
  static constexpr int VS = VC + VC_BYTES;
  static constexpr int BYTES = VS + VS_BYTES;
  static constexpr int KCHUNKS = D / 32;        // 16-byte chunks per K^ row
};

__device__ __forceinline__ v8i widen(v4i x) { return v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }

// Largest of w[0 .. n): sixteen independent loads per round trip (indices past the end repeat the
// last element, which leaves the maximum unchanged), rather than one dependent load per element.
__device__ __forceinline__ float prefix_max(const float* __restrict__ w, int n) {
  float m = -__builtin_inff();
  for (int s0 = 0; s0 < n; s0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = w[min(s0 + u, n - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) m = fmaxf(m, v[u]);
  }
  return m;
}

// Key held by LDS slot s (0..63) of a tile.  Slots 32T..32T+31 are the A rows of S^T MFMA T; in the
// 32x32 output layout, register r of lane l holds row 8(r/4) + 4(l/32) + r%4, and this map makes
// that row key 32(l/32) + 16T + r: lane l then holds all 32 keys of P block l/32 for query l%32.
__device__ __forceinline__ int slot_key(int s) {
  return 32 * ((s >> 2) & 1) + 16 * (s >> 5) + 4 * ((s >> 3) & 3) + (s & 3);
}

// three waves per SIMD for the 128-row workgroups at d = 128 (<= 168 VGPRs); the 64-row variant
// keeps more staging registers per thread and runs at two.  The split cache forward (decode:
// often one wave of a workgroup has rows) runs three stages and three waves per SIMD, so that
// six workgroups share a CU.
template <int D, int W, bool SPLIT>
constexpr int waves_per_simd() { return D == 128 ? (W == 4 || SPLIT ? 3 : 2) : 4; }

// Key tiles per barrier.  The plain and one-pass cache forward compute GT tiles from one half of
// 2 GT LDS stages while the other half is refilled with the next GT tiles, with one barrier per GT
// tiles: three when 2 x 3 stages for every workgroup the CU holds fit its 160 KB of LDS, else two.
// Measured against one barrier per tile (four stages, three tiles ahead), outputs identical: video
// shape 4.82-4.83 against 4.88-4.91 ms, causal GQA 0.858-0.860 against 0.880-0.883 ms, causal LLM
// 71.5-71.9 against 74.3-74.4 us; two tiles per barrier gained about half as much.  The split
// forward keeps one tile per barrier over three stages, which lets six of its workgroups share a CU.
template <int D, int W, bool SPLIT>
constexpr int tiles_per_step() {
  if (SPLIT) return 1;
  constexpr int wg_per_cu = 4 * waves_per_simd<D, W, SPLIT>() / W;
  return wg_per_cu * 6 * Stage<D>::BYTES <= 160 * 1024 ? 3 : 2;
}

// KV selects the cache forward: Nq new query rows per head against a cache of capacity Nk per KV
// head holding L_b valid keys for sequence b.  New row i sits at position L_b - Nq + i (causal
// masking is bottom-right aligned), and the query heads that share a KV head are packed into the
// waves' query columns, position-major (packed row = i * group + head within the group), so that
// one pass over the cache serves the whole group.  Rows that see no key give O = 0, m = -inf,
// l = 0; V^ blocks wholly past L_b take a unit scale, so that cache memory past the length,
// whatever it holds, cannot turn the zero P~ of the masked keys into NaN.
// SPLIT (with KV) runs one range of `tps` key tiles per workgroup: the running max starts at the
// largest score of the earlier ranges (from kv_max_kernel), which is exactly the running max the
// sequential loop would carry into the range, so every P~ code is the sequential one; the
// range's running max, row sum and unnormalised accumulator go to the workspace for
// kv_merge_kernel.
template <int D, int W, bool CAUSAL, bool EFQ, bool KV, bool SPLIT>
__global__ void __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(waves_per_simd<D, W, SPLIT>(), waves_per_simd<D, W, SPLIT>())))
fwd_kernel(FwdParams p) {
  using S = Stage<D>;
  constexpr int NT = 64 * W;                      // threads
  constexpr int KS_STEPS = D / 64;                // MFMA k-steps over the head dim
  constexpr int CT = D / 32;                      // 32-channel output tiles
  constexpr int GT = tiles_per_step<D, W, SPLIT>();
  constexpr int NSTAGE = SPLIT ? 3 : 2 * GT;       // LDS stages
  constexpr int PD = NSTAGE - 1;
  static_assert(NSTAGE >= 3 && NSTAGE <= 6, "stages");
  static_assert(4 * waves_per_simd<D, W, SPLIT>() / W * NSTAGE * Stage<D>::BYTES <= 160 * 1024,
                "the stages of every workgroup the intended occupancy puts on a CU fit its LDS");

  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * S::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: XCD-aware remap so that the workgroups of one head run on one XCD ----
  const int64_t G = p.Hq / p.Hkv;                 // query heads per KV head
  const int64_t nqt = KV ? (p.Nq * G + 32 * W - 1) / (32 * W) : p.N / (32 * W);
  const int64_t nsp = SPLIT ? p.splits : 1;
  const int64_t total = nqt * (KV ? p.Hkv : p.Hq) * p.B * nsp;
  int64_t id = blockIdx.x;
  int64_t sp = 0;                                 // key-tile range (split forward)
  if constexpr (SPLIT) {
    // range-major, as in kv_max_kernel: workgroup i runs on XCD i % 8, so each XCD takes the
    // same share of every sequence's ranges.  A sequence per XCD (the remap below) left the XCD
    // holding the longest cache with the most bytes to stream (1.4x the mean for lengths drawn
    // from U[N/4, N] over eight sequences).
    const int64_t ngrp = total / nsp;
    sp = id / ngrp;
    id -= sp * ngrp;
  } else if ((total & 7) == 0) {
    id = (id & 7) * (total >> 3) + (id >> 3);
  }
  int64_t bh = id / nqt;                          // (b, query head), cache forward: (b, KV head)
  int64_t qt = id - bh * nqt;
  if (CAUSAL && !SPLIT) {
    // longest rows first across all the heads of an XCD (query-tile major, heads interleaved), so
    // that the workgroups left at the end are the short ones; the heads of an XCD stay together
    const int64_t nbh = total / nqt;
    if ((total & 7) == 0 && (nbh & 7) == 0) {
      const int64_t hp = nbh >> 3;                // heads per XCD
      const int64_t M = total >> 3;               // work items per XCD
      const int64_t x = id / M, j = id - x * M;
      // rank r: longest first.  With three to four workgroups per CU (M in [3R, 4R], R = CUs per
      // XCD), a CU's first three workgroups are most of its work, and longest-first would start
      // some CUs with three long ones: there the first three dispatch rounds (one workgroup per CU
      // each) take the longest R, the shortest R, then the next R longest in ascending order, and
      // the rest follow longest first.  Measured on the causal LLM shape (M = 4R): 71.6 against
      // 73.3 us.
      constexpr int64_t R = kCuPerXcd;
      int64_t r = j;
      if (M >= 3 * R && M <= 4 * R) {
        if (j >= R && j < 2 * R) r = M - R + (j - R);
        else if (j >= 2 * R && j < 3 * R) r = 2 * R - 1 - (j - 2 * R);
        else if (j >= 3 * R) r = j - R;
      }
      bh = x * hp + r % hp;
      qt = nqt - 1 - r / hp;
    } else {
      qt = nqt - 1 - qt;
    }
  }
  int64_t b, g, qrow;                             // qrow: the lane's row in [B, Hq, Nq] order
  int64_t NK;                                     // key rows per KV head in memory
  // last visible key of the lane's row, of the wave's first and last rows, of the workgroup's
  // last row (-1: none); rows are ordered so that these limits never decrease along the rows
  int lim, lim_lo, lim_hi, lim_wg;
  int klen;                                       // valid keys (cache forward)
  bool valid = true;                              // the lane's row exists (cache forward)
  int64_t prow = 0;                               // the lane's packed row (cache forward)
  if constexpr (KV) {
    b = bh / p.Hkv;
    g = bh - b * p.Hkv;
    NK = p.Nk;
    const int64_t RK = p.Nq * G;                  // packed rows of this KV head
    const int64_t pr0 = qt * 32 * W, prw = pr0 + 32 * wave, pr = prw + l32;
    valid = pr < RK;
    prow = pr;
    const int64_t prc = min(pr, RK - 1);
    const int64_t i = prc / G;
    qrow = (b * p.Hq + g * G + (prc - i * G)) * p.Nq + i;
    const int64_t len = p.seqlens != nullptr ? min(max((int64_t)p.seqlens[b], (int64_t)0), p.Nk) : p.Nk;
    klen = (int)len;
    auto lim_of = [&](int64_t r) -> int { return (int)(CAUSAL ? min(len - p.Nq + r / G, len - 1) : len - 1); };
    lim = valid ? lim_of(prc) : -1;
    lim_lo = prw < RK ? lim_of(prw) : -1;
    lim_hi = prw < RK ? lim_of(min(prw + 31, RK - 1)) : -1;
    lim_wg = lim_of(min(pr0 + 32 * W - 1, RK - 1));
  } else {
    b = bh / p.Hq;
    const int64_t h = bh - b * p.Hq;
    g = h / G;
    NK = p.N;
    const int64_t q0 = qt * 32 * W, qw = q0 + 32 * wave, row = qw + l32;
    qrow = (b * p.Hq + h) * p.N + row;
    lim = (int)(CAUSAL ? row : p.N - 1);
    lim_lo = (int)(CAUSAL ? qw : p.N - 1);
    lim_hi = (int)(CAUSAL ? qw + 31 : p.N - 1);
    lim_wg = (int)(CAUSAL ? q0 + 32 * W - 1 : p.N - 1);
    klen = (int)p.N;
  }

  // K^ / V^ of this KV head as buffer resources: 32-bit lane offsets, the tile offset in an SGPR
  const int64_t kvh = b * p.Hkv + g;
  const auto kc_rs = make_rsrc(p.k_codes + kvh * NK * (D / 2), NK * (D / 2));
  const auto ks_rs = make_rsrc(p.k_scales + kvh * NK * (D / 32), NK * (D / 32));
  const auto vc_rs = make_rsrc(p.v_codes + kvh * D * (NK / 2), D * (NK / 2));
  const auto vs_rs = make_rsrc(p.v_scales + kvh * D * (NK / 32), D * (NK / 32));

  // ---- the wave's Q^ as the B operand of S^T = K^ Q^T (fixed for the whole kernel) ----
  v4i qb[KS_STEPS];
  int qsc;
  {
    const uint8_t* qr = p.q_codes + qrow * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS_STEPS; ++ks) qb[ks] = *reinterpret_cast<const v4i*>(qr + 16 * hi + 32 * ks);
    const uint8_t* qs = p.q_scales + qrow * (D / 32);
    qsc = (D == 128) ? (int)(qs[hi] | (qs[2 + hi] << 16)) : (int)qs[hi];
  }

  // constant A operand of the row-sum MFMA (16x16x128): row 0 sums the K-blocks holding query
  // l%16 (lanes 0-15 and 32-47), row 1 those holding query l%16 + 16 (lanes 16-31, 48-63)
  v4i ones_a;
  {
    const int r16 = lane & 15, kb = lane >> 4;
    const int on = (r16 == 0 && (kb & 1) == 0) || (r16 == 1 && (kb & 1) == 1);
    const int v = on ? 0x22222222 : 0;           // E2M1 code 2 = 1.0
    ones_a = v4i{v, v, v, v};
  }

  // ---- tile staging: direct global -> LDS loads (buffer_load ... lds), no registers ----
  // A tile is a fixed list of jobs, each one 64-lane LDS-DMA instruction writing a contiguous
  // range of the stage (lane i at +16i for 16-byte loads, at +4i for 1-4 byte loads): K^ codes in
  // 1-KB pieces, V^ codes likewise, the K^ scales, the V^ scales.  The swizzled LDS layouts are produced by choosing
  // each lane's global source.  Wave w issues jobs w, w + W, ...; every wave issues the same
  // number (JPW) per tile, the last job repeated where the list runs out (an identical rewrite).
  constexpr int KCH = S::KCHUNKS;
  constexpr int NKJ = S::KC_BYTES / 1024, NVJ = S::VC_BYTES / 1024, NVSJ = 1;
  constexpr int NJ = NKJ + NVJ + 1 + NVSJ;
  constexpr int JPW = (NJ + W - 1) / W;
  static_assert(S::KC_BYTES % 1024 == 0 && S::VC_BYTES % 1024 == 0 && S::VS_BYTES % 256 == 0, "whole jobs");
  uint32_t job_goff[JPW];                          // lane's global byte offset within tile 0
  int job_kind[JPW], job_dst[JPW];                 // wave-uniform
#pragma unroll
  for (int i = 0; i < JPW; ++i) {
    const int j = min(wave + W * i, NJ - 1);
    if (j < NKJ) {                                 // K^ codes: 16-byte chunk c of the stage
      const int c = 64 * j + lane, sl = c / KCH, cc = (c % KCH) ^ swz_small(c / KCH, KCH);
      job_kind[i] = 0; job_dst[i] = S::KC + 1024 * j;
      job_goff[i] = slot_key(sl) * (D / 2) + 16 * cc;
    } else if (j < NKJ + NVJ) {                    // V^ codes: block cc of channel ch (block-major)
      const int c = 64 * (j - NKJ) + lane, ch = c >> 1, cc = (c & 1) ^ swz_small(ch >> 1, 2);
      job_kind[i] = 1; job_dst[i] = S::VC + 1024 * (j - NKJ);
      job_goff[i] = 16 * D * cc + 16 * ch;
    } else if (j == NKJ + NVJ) {                   // K^ scales, one slot per lane
      job_kind[i] = 2; job_dst[i] = S::KS;
      job_goff[i] = slot_key(lane) * (D / 32);
    } else {                                       // V^ scales: the tile's 2d bytes, 4 per lane
      job_kind[i] = 3; job_dst[i] = S::VS;
      job_goff[i] = 4 * lane;
    }
  }
  // job kinds: 0 K^ codes, 1 V^ codes, 2 K^ scales, 3 V^ scales; a job slot whose kind is the
  // same for every wave is emitted without a branch
  auto kind_of = [](int j) constexpr { return j < NKJ ? 0 : j < NKJ + NVJ ? 1 : j == NKJ + NVJ ? 2 : 3; };
  auto issue_kind = [&](int kind, int i, int t, uint8_t* stage) {
    auto* dst = (__attribute__((address_space(3))) void*)(stage + job_dst[i]);
    if (kind == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kc_rs, dst, 16, (int)job_goff[i], t * (BC * D / 2), 0, 0);
    } else if (kind == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vc_rs, dst, 16, (int)job_goff[i], t * (BC * D / 2), 0, 0);
    } else if (kind == 2) {                        // d/32 bytes of K^ scales per slot
      if constexpr (D == 128) __builtin_amdgcn_raw_ptr_buffer_load_lds(ks_rs, dst, 4, (int)job_goff[i], t * (BC * D / 32), 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(ks_rs, dst, 2, (int)job_goff[i], t * (BC * D / 32), 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vs_rs, dst, 4, (int)job_goff[i], t * (2 * D), 0, 0);
    }
  };
  auto issue_job = [&](auto ic, int t, uint8_t* stage) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < JPW) {
      constexpr int klo = kind_of(W * i < NJ - 1 ? W * i : NJ - 1);
      constexpr int khi = kind_of(W * i + W - 1 < NJ - 1 ? W * i + W - 1 : NJ - 1);
      if constexpr (klo == khi) issue_kind(klo, i, t, stage);
      else issue_kind(job_kind[i], i, t, stage);
    }
  };
  auto issue_tile = [&](int t, uint8_t* stage) {
    t = __builtin_amdgcn_readfirstlane(t);         // tile offsets live in SGPRs
    static_assert(JPW <= 6, "job slots");
    issue_job(std::integral_constant<int, 0>{}, t, stage);
    issue_job(std::integral_constant<int, 1>{}, t, stage);
    issue_job(std::integral_constant<int, 2>{}, t, stage);
    issue_job(std::integral_constant<int, 3>{}, t, stage);
    issue_job(std::integral_constant<int, 4>{}, t, stage);
    issue_job(std::integral_constant<int, 5>{}, t, stage);
  };

  // ---- per-lane LDS read offsets (constant over tiles) ----
  int kr_off[KS_STEPS];
#pragma unroll
  for (int ks = 0; ks < KS_STEPS; ++ks)
    kr_off[ks] = S::KC + l32 * (D / 2) + 16 * ((hi + 2 * ks) ^ swz_small(l32, S::KCHUNKS));
  const int ksr_off = S::KS + 4 * l32 + hi;        // + 128 T: the lane's first block (hi) of slot l32
  const int vr_off = S::VC + l32 * 32 + 16 * (hi ^ swz_small(l32 >> 1, 2));
  const int vsr_off = S::VS + D * hi + l32;        // + 32 ct: block hi of channel 32 ct + l32

  v16f o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = v16f{};
  v4f lsum = v4f{};
  float m_run = -__builtin_inff();
  const int64_t RKs = SPLIT ? p.Nq * G : 0;       // packed rows per KV head (workspace rows)
  if constexpr (SPLIT) {                          // the running max carried into this range
    if (valid) m_run = prefix_max(p.ws_smax + (bh * RKs + prow) * nsp, (int)sp);
  }
  const float c = p.c;

  // ---- one 64-key tile: S^T, online softmax, P~ requantization, row sums and PV ----
  auto tile = [&](int t, const uint8_t* base) {
    // S^T = K^ Q^T for the two 32-key halves
    v16f sT[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      // the slot's blocks hi (k-step 0) and 2 + hi (k-step 1), one byte read each
      const int ksc0 = base[ksr_off + 128 * T];
      const v4i ka0 = *reinterpret_cast<const v4i*>(base + kr_off[0] + T * 32 * (D / 2));
      sT[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka0), widen(qb[0]), v16f{}, 4, 4, 0, ksc0, 0, qsc);
      if (KS_STEPS == 2) {
        const int ksc1 = base[ksr_off + 128 * T + 2];
        const v4i ka1 = *reinterpret_cast<const v4i*>(base + kr_off[KS_STEPS - 1] + T * 32 * (D / 2));
        sT[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(ka1), widen(qb[KS_STEPS - 1]), sT[T], 4, 4, 0,
                                                               ksc1, 2, qsc);
      }
    }
    if ((CAUSAL || KV) && t * BC + BC - 1 > lim_lo) {   // keys past a row's limit -> -inf
      const int jrel = lim - t * BC - 32 * hi;        // register r of T holds key 32 hi + 16T + r
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * T + r > jrel) sT[T][r] = -__builtin_inff();
    }
    // the lane's own block maximum (all 32 keys of block hi), then the partner lane's by one swap
    float a = fmaxf(fmaxf(sT[0][0], sT[0][1]), sT[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) a = fmaxf(fmaxf(a, sT[0][r]), sT[0][r + 1]);
    a = fmaxf(fmaxf(a, sT[0][15]), sT[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) a = fmaxf(fmaxf(a, sT[1][r]), sT[1][r + 1]);
    const float bm = fmaxf(a, sT[1][15]);
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    const float m_new = fmaxf(m_run, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
    // a row that has seen no key yet keeps m = -inf; its shift is taken as 0 (alpha = 0, p = 0)
    const float m_sh = KV ? (m_new == -__builtin_inff() ? 0.0f : m_new) : m_new;
    const float m_prev = m_run;
    const bool raised = m_new != m_prev;          // else alpha = exp2(0) = 1: nothing to rescale
    m_run = m_new;
    // E8M0 scale of the block from its max p = exp2((bm - m) c): the biased exponent of p is
    // floor((bm - m) c) + 127 (the row's own maximum gives exactly 0, i.e. p = 1); scale byte =
    // that - 2, clamped below at 1 (affects only P < 2^-124; a fully masked block gives -inf).
    const int psc = (int)__builtin_floorf(fmaxf((bm - m_sh) * c, -124.0f)) + 125;
    const float sc = __uint_as_float((uint32_t)psc << 23);
    // p = exp2(s c - m c) and E2M1 conversion against the block scale; the packed codes are
    // already the B operand of the PV MFMA (lane l: keys 32(l/32) .. +31 of query l%32)
    const float mc = m_sh * c;
    uint32_t pk[2][2];
    if constexpr (EFQ) {
      // exp-free codes: k = clamp(rne(A y + B), 0, 7) with y = x - e, x = s c - m c = log2 p and
      // e = psc - 127; one FMA per score: A y + B = s (A c) + (B - A (m c + e)).  A, B: the
      // least-squares line through (log2 v, k) of the non-zero E2M1 magnitudes v.
      constexpr float kA = 1.7470566f, kB = 2.3141184f;
      const float ac = kA * c, tb = kB - kA * (mc + (float)(psc - 127));
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          uint32_t ev = 0, od = 0;   // bytes: codes of the even / odd keys of the 8
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // v_cvt_pk_u8_f32 rounds half to even and saturates: negative values, -inf (masked
            // keys) and NaN give 0 (checked on the GPU), so only the top needs a clamp
            const float t0 = __builtin_fmaf(sT[T][8 * hw + 2 * i], ac, tb);
            const float t1 = __builtin_fmaf(sT[T][8 * hw + 2 * i + 1], ac, tb);
            ev = __builtin_amdgcn_cvt_pk_u8_f32(t0, i, ev);
            od = __builtin_amdgcn_cvt_pk_u8_f32(t1, i, od);
          }
          // y < 3 below the block's exponent bound keeps t < 3 A + B < 7.56, so every nibble is
          // at most 8; min(code, 7) for all eight at once: a nibble of 8 loses its bit 3's worth
          const uint32_t u = ev | (od << 4);
          pk[T][hw] = u - ((u >> 3) & 0x11111111u);
        }
    } else {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sT[T][8 * hw + i], c, -mc));
        uint32_t u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(e[0]), e[0], e[1], sc, 0);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, e[2], e[3], sc, 1);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, e[4], e[5], sc, 2);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, e[6], e[7], sc, 3);
        pk[T][hw] = u;
      }
    }
    }
    const v8i pb = v8i{(int)pk[0][0], (int)pk[0][1], (int)pk[1][0], (int)pk[1][1], 0, 0, 0, 0};

    // history rescale (skipped, with its exp, when no row of the wave raised its max)
    if (__builtin_amdgcn_ballot_w64(raised) != 0) {
      const float alpha = __builtin_amdgcn_exp2f((m_prev - m_sh) * c);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
      auto ah = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
      lsum[0] *= alpha;
      lsum[1] *= __uint_as_float(ah[1]);
    }
    // l += sum P~ (matrix core) and acc += P~ V^
    lsum = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(ones_a), pb, lsum, 4, 4, 0, 127, 0, psc);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const v8i va = widen(*reinterpret_cast<const v4i*>(base + vr_off + ct * 32 * 32));
      int vsc = base[vsr_off + 32 * ct];
      if constexpr (KV) vsc = t * BC + 32 * hi >= klen ? 127 : vsc;   // block wholly past the length
      o[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, o[ct], 4, 4, 0, vsc, 0, psc);
    }
  };

  // ---- tile loop: unrolled over the stages so that stage offsets are static ----
  const int ntl_all = lim_wg >= 0 ? lim_wg / BC + 1 : 0;                // workgroup-uniform
  const int tb = SPLIT ? (int)(sp * p.tps) : 0;                          // first tile of the range
  const int ntiles = SPLIT ? min((int)p.tps, ntl_all - tb) : ntl_all;    // tiles in the range
  if (SPLIT && ntiles <= 0) return;                                      // whole workgroup
  const int last_active = lim_hi >= 0 ? lim_hi / BC : -1;                // wave-uniform

  // Every barrier publishes staged tiles and frees stages: each wave first waits for its own DMAs
  // (s_waitcnt vmcnt) and its LDS reads (lgkmcnt), so that after the barrier every wave may read
  // the tiles just landed and refill the stages just read.  The asm statements also keep the
  // compiler from moving memory accesses across the barrier.
  if constexpr (!SPLIT) {
    // GT tiles per step: the step computing from one half of the stages first refills the other
    // half, freed by the barrier that ended the previous step, with the next GT tiles
    for (int k = 0; k < GT; ++k)
      if (k < ntiles) issue_tile(tb + k, smem + k * S::BYTES);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    auto group = [&](int t, auto hc) {
      constexpr int s0 = decltype(hc)::value ? GT : 0, l0 = GT - s0;
#pragma unroll
      for (int i = 0; i < GT; ++i)
        if (t + GT + i < ntiles) issue_tile(tb + t + GT + i, smem + (l0 + i) * S::BYTES);
#pragma unroll
      for (int i = 0; i < GT; ++i)
        if (t + i < ntiles && tb + t + i <= last_active) tile(tb + t + i, smem + (s0 + i) * S::BYTES);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    for (int t = 0; t < ntiles; t += 2 * GT) {
      group(t, std::integral_constant<int, 0>{});
      if (t + GT >= ntiles) break;
      group(t + GT, std::integral_constant<int, 1>{});
    }
  } else {
    // one tile per step over three stages, two tiles ahead: the barrier that ends step t publishes
    // tile t + 1 (all DMAs but the JPW that step t issued for tile t + 2 have landed) and frees the
    // stage of tile t, which step t + 1 refills
    static_assert(NSTAGE == 3, "stages");
    for (int k = 0; k < PD; ++k)
      if (k < ntiles) issue_tile(tb + k, smem + k * S::BYTES);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    static_assert(JPW <= 15, "vmcnt immediate");
    auto step = [&](int t, auto stc) {
      constexpr int st = decltype(stc)::value;
      if (t + PD < ntiles) issue_tile(tb + t + PD, smem + ((st + PD) % NSTAGE) * S::BYTES);
      if (tb + t <= last_active) tile(tb + t, smem + st * S::BYTES);
      if (t + PD < ntiles)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(JPW) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    for (int t = 0; t < ntiles; t += NSTAGE) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 >= ntiles) break;
      step(t + 1, std::integral_constant<int, 1>{});
      if (t + 2 >= ntiles) break;
      step(t + 2, std::integral_constant<int, 2>{});
    }
  }

  // ---- epilogue: gather l per query, normalise, store O (bf16), m, l ----
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lsum[0]), __float_as_uint(lsum[1]), false, false);
  auto r32 = __builtin_amdgcn_permlane32_swap(r16[0], r16[0], false, false);
  const float lrow = __uint_as_float(r32[0]);
  if constexpr (SPLIT) {                          // the range's partial results
    if (!valid) return;
    const int64_t wr = (bh * RKs + prow) * nsp + sp;
    float* orow = p.ws_o + wr * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(orow + 32 * ct + 8 * a + 4 * hi) =
            make_float4(o[ct][4 * a], o[ct][4 * a + 1], o[ct][4 * a + 2], o[ct][4 * a + 3]);
    if (hi == 0) {
      p.ws_m[wr] = m_run;
      p.ws_l[wr] = lrow;
    }
    return;
  }
  const float inv = KV ? (lrow > 0.0f ? 1.0f / lrow : 0.0f) : 1.0f / lrow;
  if (!valid) return;
  uint16_t* orow = p.o + qrow * D;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * ct + 8 * a + 4 * hi;
      uint2 w;
      w.x = pk_bf16(o[ct][4 * a + 0] * inv, o[ct][4 * a + 1] * inv);
      w.y = pk_bf16(o[ct][4 * a + 2] * inv, o[ct][4 * a + 3] * inv);
      *reinterpret_cast<uint2*>(orow + ch) = w;
    }
  if (hi == 0) {
    p.m[qrow] = m_run * p.scale_nat;
    p.l[qrow] = lrow;
  }
}

}  // namespace

}  // namespace attnfp4
