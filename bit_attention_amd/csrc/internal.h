// Internal launch interface between the C-ABI layer and the kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfp4 {

struct FwdParams {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  uint16_t* o;
  float* m;
  float* l;
  int64_t B, Hq, Hkv, N;
  float c;          // softmax_scale * log2(e): raw score -> base-2 exponent
  float scale_nat;  // softmax_scale: raw score -> natural-log units (saved m)
  // cache forward only: Nq new query rows per head, a key/value cache of capacity Nk per KV
  // head and per-sequence valid lengths (null: every sequence has Nk)
  int64_t Nq, Nk;
  const int32_t* seqlens;
  // split cache forward (see KvSplit): key tiles split into `splits` ranges of `tps` tiles; the
  // workspace regions hold, per (b, KV head, packed row, split), the split's largest visible raw
  // score, its final running max, its row sum and its unnormalised output accumulator
  int64_t splits, tps;
  float* ws_smax;
  float* ws_m;
  float* ws_l;
  float* ws_o;
};

// How the cache forward splits the key tiles across workgroups (splits == 1: one pass, no
// workspace) and the byte offsets of its workspace regions (each 256-byte aligned).
struct KvSplit {
  int64_t splits, tps;
  int64_t smax, m, l, o, total;
};
KvSplit kv_split_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d);

struct BwdParams {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const uint16_t* o;
  const uint16_t* dout;
  const float* m;
  const float* l;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  // workspace (carved by the host layer, see BwdWorkspace)
  float* rowc;      // per query row (m * log2(e), 1 / l, D = rowsum(dO * O), D / l), [B, Hq, N, 4]
  uint16_t* vb;     // V^ dequantized, bf16 [B, Hkv, N, d]
  uint16_t* kt;     // K^ dequantized and transposed, bf16 [B, Hkv, d, N]
  uint16_t* qt;     // Q^ dequantized and transposed, bf16 [B, Hq, d, N]
  uint16_t* dot;    // dO transposed, each query row times its 1/l, bf16 [B, Hq, d, N]
  // the d = 128 dK/dV path reads row-major copies instead (same workspace regions as qt, dot):
  uint16_t* qb;     // Q^ dequantized, bf16 [B, Hq, N, d]
  uint16_t* dos;    // dO times each row's 1/l, bf16 [B, Hq, N, d]
  int64_t B, Hq, Hkv, N, d;
  int causal;
  float c;          // softmax_scale * log2(e)
  float scale_nat;  // softmax_scale
};

// Byte offsets of the backward's workspace regions (each 256-byte aligned).
struct BwdWorkspace {
  int64_t rowc, vb, kt, qt, dot, total;
};
BwdWorkspace bwd_workspace_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d);

// NVFP4-style forward: the operands dequantized to fp16 (E2M1 * E4M3 scale, exact) in the
// workspace, and the device-resident fp32 tensor scales.
struct NvFwdParams {
  const uint16_t* qb;   // Q^ / G_Q, fp16 [B, Hq, N, d]
  const uint16_t* kb;   // K^ / G_K, fp16 [B, Hkv, N, d]
  const uint16_t* vt;   // V^ / G_V transposed, fp16 [B, Hkv, d, N]
  const float* q_ts;    // tensor scales G (first float of each attn_fp4_nv_quantize output)
  const float* k_ts;
  const float* v_ts;
  uint16_t* o;
  float* m;
  float* l;
  int64_t B, Hq, Hkv, N;
  float scale_nat;      // softmax_scale
};

struct NvWorkspace {
  int64_t qb, kb, vt, total;
};
NvWorkspace nv_fwd_workspace_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d);

hipError_t launch_nv_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int axis, void* codes, void* scales,
                              float* ts, hipStream_t stream);
hipError_t launch_nv_fwd(const NvFwdParams& p, const void* q_codes, const void* q_scales, const void* k_codes,
                         const void* k_scales, const void* v_codes, const void* v_scales, int d, bool causal,
                         hipStream_t stream);

hipError_t launch_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int axis, void* codes,
                           void* scales, hipStream_t stream);
hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream);
hipError_t launch_fwd_kvcache(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream);
// the split form (p.splits > 1): max pass, split forward, merge
hipError_t launch_fwd_kvcache_split(const FwdParams& p, int d, bool causal, bool efq, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace attnfp4
