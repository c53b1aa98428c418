// C-ABI host layer of libattnfp4: argument validation, device check, launch.
// No allocation, no synchronisation, no printing; every error is a status code.
#include <string.h>

#include <cmath>

#include "../../include/attn_fp4.h"
#include "internal.h"

namespace {

constexpr int32_t kAbiVersion = 7;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device cache of the "is gfx950" check: 0 unknown, 1 yes, 2 no.
int g_arch_ok[64];

int32_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_FP4_E_HIP;
  if (dev < 0) return ATTN_FP4_E_HIP;
  if (dev < 64 && g_arch_ok[dev] == 1) return ATTN_FP4_OK;
  if (dev < 64 && g_arch_ok[dev] == 2) return ATTN_FP4_E_UNSUPPORTED_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_FP4_E_HIP;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_ok[dev] = ok ? 1 : 2;
  return ok ? ATTN_FP4_OK : ATTN_FP4_E_UNSUPPORTED_DEVICE;
}

float resolve_scale(float s, int64_t d) { return s > 0.0f ? s : (float)(1.0 / std::sqrt((double)d)); }

int32_t check_dims(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return ATTN_FP4_E_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_FP4_E_INVALID_ARG;
  if (N % 64 != 0 || Hq % Hkv != 0) return ATTN_FP4_E_INVALID_ARG;
  // grid sizes: (N / 64) * Hq * B workgroups must fit a 32-bit grid dimension
  if ((N / 64) * Hq * B > (int64_t)0x7FFFFFFF) return ATTN_FP4_E_INVALID_ARG;
  return ATTN_FP4_OK;
}

}  // namespace

extern "C" {

int32_t attn_fp4_abi_version(void) { return kAbiVersion; }

const char* attn_fp4_status_string(int32_t status) {
  switch (status) {
    case ATTN_FP4_OK: return "ok";
    case ATTN_FP4_E_INVALID_ARG: return "invalid argument (pointer, alignment, shape or enum)";
    case ATTN_FP4_E_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 / MI355X required)";
    case ATTN_FP4_E_UNSUPPORTED: return "unsupported configuration in this build";
    case ATTN_FP4_E_HIP: return "HIP runtime or kernel launch error";
    case ATTN_FP4_E_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int32_t attn_fp4_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int32_t axis, void* codes,
                          void* scales, void* stream) {
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return ATTN_FP4_E_INVALID_ARG;
  if (bh <= 0 || n <= 0 || d <= 0) return ATTN_FP4_E_INVALID_ARG;
  if (axis != 0 && axis != 1) return ATTN_FP4_E_INVALID_ARG;
  if (d % 32 != 0) return ATTN_FP4_E_INVALID_ARG;
  // axis 0: one thread per four 8-element groups; axis 1: one thread per (32-token block,
  // channel pair); each grid must fit 32 bits
  if (axis == 0 && (bh * n * (d / 8) + 1023) / 1024 > 0x7FFFFFFF) return ATTN_FP4_E_INVALID_ARG;
  if (axis == 1 && (n % 32 != 0 || (bh * (n / 32) * (d / 2) + 255) / 256 > 0x7FFFFFFF)) return ATTN_FP4_E_INVALID_ARG;
  int32_t st = check_device();
  if (st != ATTN_FP4_OK) return st;
  hipError_t e = attnfp4::launch_quantize(x, bh, n, d, axis, codes, scales, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_FP4_OK : ATTN_FP4_E_HIP;
}

int32_t attn_fp4_fwd(const attn_fp4_fwd_args* a, void* stream) {
  if (a == nullptr) return ATTN_FP4_E_INVALID_ARG;
  int32_t st = check_dims(a->B, a->Hq, a->Hkv, a->N, a->d);
  if (st != ATTN_FP4_OK) return st;
  const void* ptrs[] = {a->q_codes, a->q_scales, a->k_codes, a->k_scales, a->v_codes,
                        a->v_scales, a->o, a->m, a->l};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_FP4_E_INVALID_ARG;
  if (!(a->softmax_scale <= 0.0f || std::isfinite(a->softmax_scale))) return ATTN_FP4_E_INVALID_ARG;
  if (a->p_rule != ATTN_FP4_P_EXP && a->p_rule != ATTN_FP4_P_EFQ) return ATTN_FP4_E_INVALID_ARG;
  // the kernels address one KV head's K^ / V^ codes with 32-bit buffer offsets
  if (a->N * a->d / 2 > (int64_t)0x7FFFFFFF) return ATTN_FP4_E_UNSUPPORTED;
  st = check_device();
  if (st != ATTN_FP4_OK) return st;
  attnfp4::FwdParams p;
  p.q_codes = (const uint8_t*)a->q_codes;
  p.q_scales = (const uint8_t*)a->q_scales;
  p.k_codes = (const uint8_t*)a->k_codes;
  p.k_scales = (const uint8_t*)a->k_scales;
  p.v_codes = (const uint8_t*)a->v_codes;
  p.v_scales = (const uint8_t*)a->v_scales;
  p.o = (uint16_t*)a->o;
  p.m = a->m;
  p.l = a->l;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.N = a->N;
  p.Nq = a->N;
  p.Nk = a->N;
  p.seqlens = nullptr;
  p.splits = 1;
  p.tps = a->N / 64;
  p.ws_smax = p.ws_m = p.ws_l = p.ws_o = nullptr;
  const double s = resolve_scale(a->softmax_scale, a->d);
  p.c = (float)(s * 1.4426950408889634);
  p.scale_nat = (float)s;
  hipError_t e = attnfp4::launch_fwd(p, (int)a->d, a->causal != 0, a->p_rule == ATTN_FP4_P_EFQ, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_FP4_OK : ATTN_FP4_E_HIP;
}

static int32_t check_kvcache_dims(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return ATTN_FP4_E_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_FP4_E_INVALID_ARG;
  if (Nk % 64 != 0 || Hq % Hkv != 0) return ATTN_FP4_E_INVALID_ARG;
  // the grid: at most one workgroup per 64 packed query rows (times the splits)
  if ((Nq * (Hq / Hkv) + 63) / 64 * Hkv * B * (Nk / 64) > (int64_t)0x7FFFFFFF) return ATTN_FP4_E_INVALID_ARG;
  // the kernels address one KV head's cache codes with 32-bit buffer offsets
  if (Nk * d / 2 > (int64_t)0x7FFFFFFF) return ATTN_FP4_E_UNSUPPORTED;
  return ATTN_FP4_OK;
}

int64_t attn_fp4_fwd_kvcache_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  if (check_kvcache_dims(B, Hq, Hkv, Nq, Nk, d) != ATTN_FP4_OK) return -1;
  return attnfp4::kv_split_plan(B, Hq, Hkv, Nq, Nk, d).total;
}

// The cache forward with the split workspace given explicitly (workspace == nullptr: one pass).
static int32_t fwd_kvcache_impl(const attn_fp4_fwd_kvcache_args* a, void* workspace, int64_t workspace_bytes,
                                void* stream) {
  if (a == nullptr) return ATTN_FP4_E_INVALID_ARG;
  int32_t st0 = check_kvcache_dims(a->B, a->Hq, a->Hkv, a->Nq, a->Nk, a->d);
  if (st0 != ATTN_FP4_OK) return st0;
  const void* ptrs[] = {a->q_codes, a->q_scales, a->k_codes, a->k_scales, a->v_codes,
                        a->v_scales, a->o, a->m, a->l};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_FP4_E_INVALID_ARG;
  if (a->seqlens_k != nullptr && (reinterpret_cast<uintptr_t>(a->seqlens_k) & 3u) != 0) return ATTN_FP4_E_INVALID_ARG;
  if (!(a->softmax_scale <= 0.0f || std::isfinite(a->softmax_scale))) return ATTN_FP4_E_INVALID_ARG;
  if (a->p_rule != ATTN_FP4_P_EXP && a->p_rule != ATTN_FP4_P_EFQ) return ATTN_FP4_E_INVALID_ARG;
  const attnfp4::KvSplit ks = attnfp4::kv_split_plan(a->B, a->Hq, a->Hkv, a->Nq, a->Nk, a->d);
  if (workspace != nullptr && ks.splits > 1 &&
      ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < ks.total))
    return ATTN_FP4_E_WORKSPACE;
  int32_t st = check_device();
  if (st != ATTN_FP4_OK) return st;
  attnfp4::FwdParams p;
  p.q_codes = (const uint8_t*)a->q_codes;
  p.q_scales = (const uint8_t*)a->q_scales;
  p.k_codes = (const uint8_t*)a->k_codes;
  p.k_scales = (const uint8_t*)a->k_scales;
  p.v_codes = (const uint8_t*)a->v_codes;
  p.v_scales = (const uint8_t*)a->v_scales;
  p.o = (uint16_t*)a->o;
  p.m = a->m;
  p.l = a->l;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.N = 0;
  p.Nq = a->Nq;
  p.Nk = a->Nk;
  p.seqlens = a->seqlens_k;
  p.splits = 1;
  p.tps = a->Nk / 64;
  p.ws_smax = p.ws_m = p.ws_l = p.ws_o = nullptr;
  if (workspace != nullptr && ks.splits > 1) {
    uint8_t* w = (uint8_t*)workspace;
    p.splits = ks.splits;
    p.tps = ks.tps;
    p.ws_smax = (float*)(w + ks.smax);
    p.ws_m = (float*)(w + ks.m);
    p.ws_l = (float*)(w + ks.l);
    p.ws_o = (float*)(w + ks.o);
  }
  const double s = resolve_scale(a->softmax_scale, a->d);
  p.c = (float)(s * 1.4426950408889634);
  p.scale_nat = (float)s;
  hipError_t e = attnfp4::launch_fwd_kvcache(p, (int)a->d, a->causal != 0, a->p_rule == ATTN_FP4_P_EFQ,
                                             (hipStream_t)stream);
  return e == hipSuccess ? ATTN_FP4_OK : ATTN_FP4_E_HIP;
}

int32_t attn_fp4_fwd_kvcache(const attn_fp4_fwd_kvcache_args* a, void* stream) {
  if (a == nullptr) return ATTN_FP4_E_INVALID_ARG;
  return fwd_kvcache_impl(a, a->workspace, a->workspace_bytes, stream);
}

// ---- the cache forward for callers that cannot allocate ----
// Its split workspace is this file-scope device array: one copy on every GPU the library runs on,
// held until the process ends.  In host code the array's name is only a handle; its device
// address on the current GPU comes from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) uint8_t scratch[ATTN_FP4_KVCACHE_SCRATCH_BYTES];
static void* g_scratch[64];   // per device: the array's device address (null until looked up)

static int32_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_FP4_E_HIP;
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return ATTN_FP4_E_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return ATTN_FP4_OK;
}

int32_t attn_fp4_fwd_kvcache_noalloc(const attn_fp4_fwd_kvcache_args* a, void* stream) {
  if (a == nullptr) return ATTN_FP4_E_INVALID_ARG;
  int32_t st = check_kvcache_dims(a->B, a->Hq, a->Hkv, a->Nq, a->Nk, a->d);
  if (st != ATTN_FP4_OK) return st;
  const attnfp4::KvSplit ks = attnfp4::kv_split_plan(a->B, a->Hq, a->Hkv, a->Nq, a->Nk, a->d);
  if (ks.splits <= 1) return fwd_kvcache_impl(a, nullptr, 0, stream);   // one pass: no workspace
  if (ks.total > (int64_t)ATTN_FP4_KVCACHE_SCRATCH_BYTES) return ATTN_FP4_E_WORKSPACE;
  st = check_device();
  if (st != ATTN_FP4_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != ATTN_FP4_OK) return st;
  return fwd_kvcache_impl(a, ws, ATTN_FP4_KVCACHE_SCRATCH_BYTES, stream);
}

int64_t attn_fp4_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
  if (check_dims(B, Hq, Hkv, N, d) != ATTN_FP4_OK) return -1;
  return attnfp4::bwd_workspace_layout(B, Hq, Hkv, N, d).total;
}

int32_t attn_fp4_bwd_recompute(const attn_fp4_bwd_args* a, void* stream) {
  if (a == nullptr) return ATTN_FP4_E_INVALID_ARG;
  int32_t st = check_dims(a->B, a->Hq, a->Hkv, a->N, a->d);
  if (st != ATTN_FP4_OK) return st;
  const void* ptrs[] = {a->q_codes, a->q_scales, a->k_codes, a->k_scales, a->v_codes, a->v_scales,
                        a->o, a->do_, a->m, a->l, a->dq, a->dk, a->dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_FP4_E_INVALID_ARG;
  if (!(a->softmax_scale <= 0.0f || std::isfinite(a->softmax_scale))) return ATTN_FP4_E_INVALID_ARG;
  const attnfp4::BwdWorkspace ws = attnfp4::bwd_workspace_layout(a->B, a->Hq, a->Hkv, a->N, a->d);
  if (a->workspace == nullptr || (reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0 ||
      a->workspace_bytes < ws.total)
    return ATTN_FP4_E_WORKSPACE;
  if (a->B * a->Hq > 65535) return ATTN_FP4_E_INVALID_ARG;   // grid z of the transposes
  // the kernels address one KV head's query-head group of bf16 [N, d] tensors with 32-bit offsets
  if ((a->Hq / a->Hkv) * a->N * a->d * 2 > (int64_t)0x7FFFFFFF) return ATTN_FP4_E_UNSUPPORTED;
  st = check_device();
  if (st != ATTN_FP4_OK) return st;
  attnfp4::BwdParams p;
  p.q_codes = (const uint8_t*)a->q_codes;
  p.q_scales = (const uint8_t*)a->q_scales;
  p.k_codes = (const uint8_t*)a->k_codes;
  p.k_scales = (const uint8_t*)a->k_scales;
  p.v_codes = (const uint8_t*)a->v_codes;
  p.v_scales = (const uint8_t*)a->v_scales;
  p.o = (const uint16_t*)a->o;
  p.dout = (const uint16_t*)a->do_;
  p.m = a->m;
  p.l = a->l;
  p.dq = (uint16_t*)a->dq;
  p.dk = (uint16_t*)a->dk;
  p.dv = (uint16_t*)a->dv;
  uint8_t* w = (uint8_t*)a->workspace;
  p.rowc = (float*)(w + ws.rowc);
  p.vb = (uint16_t*)(w + ws.vb);
  p.kt = (uint16_t*)(w + ws.kt);
  p.qt = (uint16_t*)(w + ws.qt);
  p.dot = (uint16_t*)(w + ws.dot);
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.N = a->N;
  p.d = a->d;
  p.causal = a->causal != 0;
  const double s = resolve_scale(a->softmax_scale, a->d);
  p.c = (float)(s * 1.4426950408889634);
  p.scale_nat = (float)s;
  hipError_t e = attnfp4::launch_bwd(p, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return ATTN_FP4_E_UNSUPPORTED;
  return e == hipSuccess ? ATTN_FP4_OK : ATTN_FP4_E_HIP;
}

int32_t attn_fp4_nv_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int32_t axis, void* codes,
                             void* scales, float* tensor_scale, void* stream) {
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return ATTN_FP4_E_INVALID_ARG;
  if (tensor_scale == nullptr || (reinterpret_cast<uintptr_t>(tensor_scale) & 7u) != 0) return ATTN_FP4_E_INVALID_ARG;
  if (bh <= 0 || n <= 0 || d <= 0 || d % 32 != 0) return ATTN_FP4_E_INVALID_ARG;
  if (axis != 0 && axis != 1) return ATTN_FP4_E_INVALID_ARG;
  if (axis == 1 && (n % 16 != 0 || bh > 65535 || d / 32 > 65535 || (n + 127) / 128 > 0x7FFFFFFF))
    return ATTN_FP4_E_INVALID_ARG;
  int32_t st = check_device();
  if (st != ATTN_FP4_OK) return st;
  hipError_t e = attnfp4::launch_nv_quantize(x, bh, n, d, axis, codes, scales, tensor_scale, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_FP4_OK : ATTN_FP4_E_HIP;
}

int64_t attn_fp4_nv_fwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
  if (check_dims(B, Hq, Hkv, N, d) != ATTN_FP4_OK) return -1;
  return attnfp4::nv_fwd_workspace_layout(B, Hq, Hkv, N, d).total;
}

int32_t attn_fp4_nv_fwd(const attn_fp4_nv_fwd_args* a, void* stream) {
  if (a == nullptr) return ATTN_FP4_E_INVALID_ARG;
  int32_t st = check_dims(a->B, a->Hq, a->Hkv, a->N, a->d);
  if (st != ATTN_FP4_OK) return st;
  const void* ptrs[] = {a->q_codes, a->q_scales, a->k_codes, a->k_scales, a->v_codes,
                        a->v_scales, a->o, a->m, a->l};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_FP4_E_INVALID_ARG;
  const float* ts[] = {a->q_tensor_scale, a->k_tensor_scale, a->v_tensor_scale};
  for (const float* t : ts)
    if (t == nullptr || (reinterpret_cast<uintptr_t>(t) & 7u) != 0) return ATTN_FP4_E_INVALID_ARG;
  if (!(a->softmax_scale <= 0.0f || std::isfinite(a->softmax_scale))) return ATTN_FP4_E_INVALID_ARG;
  const attnfp4::NvWorkspace ws = attnfp4::nv_fwd_workspace_layout(a->B, a->Hq, a->Hkv, a->N, a->d);
  if (a->workspace == nullptr || (reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0 ||
      a->workspace_bytes < ws.total)
    return ATTN_FP4_E_WORKSPACE;
  // the kernel addresses one KV head's fp16 [N, d] operands with 32-bit buffer offsets
  if (a->N * a->d * 2 > (int64_t)0x7FFFFFFF) return ATTN_FP4_E_UNSUPPORTED;
  st = check_device();
  if (st != ATTN_FP4_OK) return st;
  uint8_t* w = (uint8_t*)a->workspace;
  attnfp4::NvFwdParams p;
  p.qb = (const uint16_t*)(w + ws.qb);
  p.kb = (const uint16_t*)(w + ws.kb);
  p.vt = (const uint16_t*)(w + ws.vt);
  p.q_ts = a->q_tensor_scale;
  p.k_ts = a->k_tensor_scale;
  p.v_ts = a->v_tensor_scale;
  p.o = (uint16_t*)a->o;
  p.m = a->m;
  p.l = a->l;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.N = a->N;
  p.scale_nat = resolve_scale(a->softmax_scale, a->d);
  hipError_t e = attnfp4::launch_nv_fwd(p, a->q_codes, a->q_scales, a->k_codes, a->k_scales, a->v_codes, a->v_scales,
                                        (int)a->d, a->causal != 0, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_FP4_OK : ATTN_FP4_E_HIP;
}

}  // extern "C"
