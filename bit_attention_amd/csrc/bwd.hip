// Attn-QAT backward with FP4 recomputation of the scores (gfx950).  Placeholder launch until the
// kernels land: reports "not supported" so the C-ABI returns ATTN_FP4_E_UNSUPPORTED.
#include "common.h"
#include "internal.h"

namespace attnfp4 {

int64_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t N, int64_t d) {
  const int64_t delta = ((B * Hq * N * 4 + 255) / 256) * 256;
  const int64_t dq = ((B * Hq * N * d * 4 + 255) / 256) * 256;
  return delta + dq;
}

hipError_t launch_bwd(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attnfp4
