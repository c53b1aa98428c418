// Launches of the MXFP4 forward kernel (fwd_kernel.h): the plain forward and the one-pass cache
// forward, and the split plan of the cache forward (whose passes are in fwd_split.hip).  This file
// is compiled with LLVM's iterative ILP scheduler (bit_attention_amd/build.py).
#include "fwd_kernel.h"

namespace attnfp4 {

namespace {

template <int D, int W, bool CAUSAL, bool EFQ, bool KV>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int64_t blocks = KV ? ((p.Nq * (p.Hq / p.Hkv) + 32 * W - 1) / (32 * W)) * p.Hkv * p.B
                            : (p.N / (32 * W)) * p.Hq * p.B;
  hipLaunchKernelGGL((fwd_kernel<D, W, CAUSAL, EFQ, KV, false>), dim3((unsigned)blocks), dim3(64 * W), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool EFQ, bool KV>
hipError_t launch_d(const FwdParams& p, bool causal, hipStream_t stream) {
  // four waves (128 rows) per workgroup when the rows tile evenly (plain forward) or there are
  // enough of them (cache forward), else two
  const bool w4 = KV ? p.Nq * (p.Hq / p.Hkv) >= 256 : p.N % 128 == 0;
  if (w4) return causal ? launch<D, 4, true, EFQ, KV>(p, stream) : launch<D, 4, false, EFQ, KV>(p, stream);
  return causal ? launch<D, 2, true, EFQ, KV>(p, stream) : launch<D, 2, false, EFQ, KV>(p, stream);
}

template <bool KV>
hipError_t launch_any(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream) {
  if (efq) return d == 128 ? launch_d<128, true, KV>(p, causal, stream) : launch_d<64, true, KV>(p, causal, stream);
  return d == 128 ? launch_d<128, false, KV>(p, causal, stream) : launch_d<64, false, KV>(p, causal, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream) {
  return launch_any<false>(p, d, causal, efq, stream);
}

hipError_t launch_fwd_kvcache(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream) {
  if (p.splits > 1) return launch_fwd_kvcache_split(p, d, causal, efq, stream);
  return launch_any<true>(p, d, causal, efq, stream);
}

// Split the key tiles when the one-pass launch would leave the chip mostly idle: fewer than 256
// workgroups of 64 packed rows (decode, short chunks).  Aim at about 1024 workgroups per pass (four
// per CU; measured best for decode against 512, 768, 1280, 1536, 2048 and 4096: fewer, longer
// ranges keep each workgroup's loads streaming, more ranges add fixed costs), at least four tiles
// per range.
KvSplit kv_split_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  KvSplit k{1, Nk / 64, 0, 0, 0, 0, 0};
  const int64_t RK = Nq * (Hq / Hkv);
  const int64_t base = (RK + 63) / 64 * Hkv * B;
  const int64_t ntc = Nk / 64;
  if (base >= 256 || ntc < 8) return k;
  int64_t s = min((1024 + base - 1) / base, ntc / 4);
  if (s < 2) return k;
  k.tps = (ntc + s - 1) / s;
  k.splits = (ntc + k.tps - 1) / k.tps;
  if (k.splits < 2) return KvSplit{1, ntc, 0, 0, 0, 0, 0};
  const int64_t rows = B * Hkv * k.splits * RK;
  auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  k.smax = 0;
  k.m = up(k.smax + rows * 4);
  k.l = up(k.m + rows * 4);
  k.o = up(k.l + rows * 4);
  k.total = up(k.o + rows * d * 4);
  return k;
}

}  // namespace attnfp4
