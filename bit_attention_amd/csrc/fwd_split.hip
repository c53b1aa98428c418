// The split cache forward (decode, short chunks): the max pass, the split forward kernel
// (fwd_kernel.h with SPLIT) and the merge.  Compiled with the default scheduler, which measured
// faster for these kernels than the iterative ILP one used for fwd.hip.
#include "fwd_kernel.h"

namespace attnfp4 {

namespace {

// ---- split cache forward, pass 1: the largest visible raw score per (split, packed row) ----
// Workgroups of two waves take 64 packed rows and one range of key tiles, as the split forward
// does (when the workgroup has at most 32 rows, both waves take them and alternate tiles).  K^ is
// read straight into the MFMA A operand, one tile ahead (no LDS; keys in natural order: the
// maximum does not depend on where a key sits), and the scores are the forward's, bit for bit
// (same operands, scales and k-step order).  A row group's last range is not run: no range after
// it reads its maximum.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(128) kv_max_kernel(FwdParams p) {
  constexpr int KS_STEPS = D / 64;
  __shared__ float xmax[32];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t G = p.Hq / p.Hkv, RK = p.Nq * G, nqt = (RK + 63) / 64, nsp = p.splits;
  // consecutive workgroups take the same range of different row groups, so that the early ranges
  // (which every sequence has) and the late ones (which only long sequences have) spread evenly
  const int64_t ngrp = nqt * p.Hkv * p.B;
  const int64_t sp = blockIdx.x / ngrp;
  const int64_t id = blockIdx.x - sp * ngrp;
  const int64_t bh = id / nqt, qt = id - bh * nqt;
  const int64_t b = bh / p.Hkv, g = bh - b * p.Hkv;
  const int64_t pr0 = qt * 64;
  const bool share = RK - pr0 <= 32;              // one row block, two waves over the tiles
  const int64_t prw = pr0 + (share ? 0 : 32 * wave), pr = prw + l32;
  const bool valid = pr < RK;
  const int64_t prc = min(pr, RK - 1);
  const int64_t i = prc / G;
  const int64_t qrow = (b * p.Hq + g * G + (prc - i * G)) * p.Nq + i;
  const int64_t len = p.seqlens != nullptr ? min(max((int64_t)p.seqlens[b], (int64_t)0), p.Nk) : p.Nk;
  auto lim_of = [&](int64_t r) -> int { return (int)(CAUSAL ? min(len - p.Nq + r / G, len - 1) : len - 1); };
  const int lim = valid ? lim_of(prc) : -1;
  const int lim_lo = prw < RK ? lim_of(prw) : -1;
  const int lim_hi = prw < RK ? lim_of(min(prw + 31, RK - 1)) : -1;
  const int lim_wg = lim_of(min(pr0 + 63, RK - 1));
  const int ntl_all = lim_wg >= 0 ? lim_wg / 64 + 1 : 0;
  const int tb = (int)(sp * p.tps);
  // the group's last range (and any range past it) is skipped: the split forward of range s reads
  // only the maxima of ranges 0 .. s - 1 (workgroup-uniform)
  if (ntl_all <= tb + (int)p.tps) return;
  const int te = min(tb + (int)p.tps, min(ntl_all, lim_hi >= 0 ? lim_hi / 64 + 1 : 0));
  const int tstep = share ? 2 : 1;
  float mx = -__builtin_inff();
  const int t0 = tb + (share ? wave : 0);
  if (t0 < te) {
    v4i qb[KS_STEPS];
    const uint8_t* qr = p.q_codes + qrow * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS_STEPS; ++ks) qb[ks] = *reinterpret_cast<const v4i*>(qr + 16 * hi + 32 * ks);
    const uint8_t* qs = p.q_scales + qrow * (D / 32);
    const int qsc = (D == 128) ? (int)(qs[hi] | (qs[2 + hi] << 16)) : (int)qs[hi];
    const int64_t kvh = b * p.Hkv + g;
    const auto kc_rs = make_rsrc(p.k_codes + kvh * p.Nk * (D / 2), p.Nk * (D / 2));
    const auto ks_rs = make_rsrc(p.k_scales + kvh * p.Nk * (D / 32), p.Nk * (D / 32));
    // A row l32 of half T is key 64 t + 32 T + l32
    struct Ops { v4i ka[2][KS_STEPS]; int ksc[2]; };
    auto load = [&](int t, Ops& o) {
      const int tt = __builtin_amdgcn_readfirstlane(t);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const int key = 32 * T + l32;
        if constexpr (D == 128)
          o.ksc[T] = (int)((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ks_rs, 4 * key, tt * 256, 0) >> (8 * hi));
        else
          o.ksc[T] = (int)__builtin_amdgcn_raw_buffer_load_b8(ks_rs, 2 * key + hi, tt * 128, 0);
#pragma unroll
        for (int ks = 0; ks < KS_STEPS; ++ks)
          o.ka[T][ks] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                    kc_rs, key * (D / 2) + 32 * ks + 16 * hi, tt * (64 * D / 2), 0));
      }
    };
    // tile t from cur while the wave's next tile is loaded into nxt: two buffers, the loop
    // unrolled by two (no buffer copies), the load unconditional (the last tile loads itself once
    // more), so that no wait before a use of cur has to cover the load just issued
    auto tile_max = [&](int t, const Ops& cur, Ops& nxt) __attribute__((always_inline)) {
      load(min(t + tstep, te - 1), nxt);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        v16f acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(cur.ka[T][0]), widen(qb[0]), v16f{}, 4, 4, 0,
                                                                   cur.ksc[T], 0, qsc);
        if constexpr (KS_STEPS == 2)
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(cur.ka[T][1]), widen(qb[1]), acc, 4, 4, 2,
                                                                cur.ksc[T], 2, qsc);
        // register r holds key 64 t + 32 T + 8 (r / 4) + 4 hi + r % 4 of query l32
        if (t * 64 + 63 > lim_lo) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t * 64 + 32 * T + 8 * (r >> 2) + 4 * hi + (r & 3) > lim) acc[r] = -__builtin_inff();
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
      }
    };
    Ops ba, bb;
    load(t0, ba);
    for (int t = t0; t < te; t += 2 * tstep) {
      tile_max(t, ba, bb);
      if (t + tstep >= te) break;
      tile_max(t + tstep, bb, ba);
    }
  }
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  if (share) {                                    // combine the two waves' tiles
    if (wave == 1 && hi == 0) xmax[l32] = mx;
    __syncthreads();
    if (wave == 1) return;
    mx = fmaxf(mx, xmax[l32]);
  }
  if (valid && hi == 0) p.ws_smax[(bh * RK + pr) * nsp + sp] = mx;
}

// ---- split cache forward, pass 3: merge the ranges' partial results into O, m, l ----
// One workgroup per packed row; the partial results of a row are contiguous ([row][range] and
// [row][range][d]).  With M the largest running max over the ranges, range s contributes
// exp2((m_s - M) c) times its accumulator and row sum: the sequential loop's history rescaling
// written as one factor per range.  Each wave takes every fourth range.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) kv_merge_kernel(FwdParams p) {
  constexpr int CPL = D / 64;                     // channels per lane
  __shared__ float red_o[4][D];
  __shared__ float red_l[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t G = p.Hq / p.Hkv, RK = p.Nq * G, nsp = p.splits;
  const int64_t rid = blockIdx.x;
  const int64_t bh = rid / RK, pr = rid - bh * RK;
  const int64_t b = bh / p.Hkv, g = bh - b * p.Hkv;
  const int64_t i = pr / G;
  const int64_t qrow = (b * p.Hq + g * G + (pr - i * G)) * p.Nq + i;
  // the ranges the split forward ran for this row's workgroup (64 packed rows)
  const int64_t len = p.seqlens != nullptr ? min(max((int64_t)p.seqlens[b], (int64_t)0), p.Nk) : p.Nk;
  const int64_t last = min((pr / 64) * 64 + 63, RK - 1);
  const int64_t lim_wg = CAUSAL ? min(len - p.Nq + last / G, len - 1) : len - 1;
  const int nr = lim_wg >= 0 ? (int)((lim_wg / 64) / p.tps + 1) : 0;
  const float* wm = p.ws_m + rid * nsp;
  const float* wl = p.ws_l + rid * nsp;
  const float* wo = p.ws_o + rid * nsp * D + CPL * lane;
  const float M = prefix_max(wm, nr);
  float acc[CPL] = {};
  float lt = 0.0f;
  if (M != -__builtin_inff()) {
#pragma unroll 4
    for (int s = wave; s < nr; s += 4) {
      const float w = __builtin_amdgcn_exp2f((wm[s] - M) * p.c);
      lt += w * wl[s];
#pragma unroll
      for (int k = 0; k < CPL; ++k) acc[k] += w * wo[(int64_t)s * D + k];
    }
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k) red_o[wave][CPL * lane + k] = acc[k];
  if (lane == 0) red_l[wave] = lt;
  __syncthreads();
  if (wave != 0) return;
  lt = red_l[0] + red_l[1] + red_l[2] + red_l[3];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int ch = CPL * lane + k;
    acc[k] = red_o[0][ch] + red_o[1][ch] + red_o[2][ch] + red_o[3][ch];
  }
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  uint16_t* orow = p.o + qrow * D + CPL * lane;
  if constexpr (CPL == 2) *reinterpret_cast<uint32_t*>(orow) = pk_bf16(acc[0] * inv, acc[1] * inv);
  else orow[0] = (uint16_t)(pk_bf16(acc[0] * inv, 0.0f) & 0xFFFFu);
  if (lane == 0) {
    p.m[qrow] = M * p.scale_nat;
    p.l[qrow] = lt;
  }
}

template <int D, bool CAUSAL, bool EFQ>
hipError_t launch_split(const FwdParams& p, hipStream_t stream) {
  const int64_t RK = p.Nq * (p.Hq / p.Hkv);
  const int64_t wgs = (RK + 63) / 64 * p.Hkv * p.B * p.splits;
  hipLaunchKernelGGL((kv_max_kernel<D, CAUSAL>), dim3((unsigned)wgs), dim3(128), 0, stream, p);
  hipLaunchKernelGGL((fwd_kernel<D, 2, CAUSAL, EFQ, true, true>), dim3((unsigned)wgs), dim3(128), 0, stream, p);
  const int64_t rows = RK * p.Hkv * p.B;
  hipLaunchKernelGGL((kv_merge_kernel<D, CAUSAL>), dim3((unsigned)rows), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const FwdParams& p, bool causal, bool efq, hipStream_t stream) {
  if (causal) return efq ? launch_split<D, true, true>(p, stream) : launch_split<D, true, false>(p, stream);
  return efq ? launch_split<D, false, true>(p, stream) : launch_split<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd_kvcache_split(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream) {
  return d == 128 ? launch_split_d<128>(p, causal, efq, stream) : launch_split_d<64>(p, causal, efq, stream);
}

}  // namespace attnfp4
