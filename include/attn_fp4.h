/*
 * attn_fp4.h -- C ABI of libattnfp4.so: 4-bit (MXFP4) FlashAttention-style
 * attention for AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *  - Attn-QAT: 4-Bit Attention With Quantization-Aware Training (abstract):
 *    an FP4 attention forward, and a backward that recomputes the attention
 *    scores with the same low-precision QK^T and takes the D term of the
 *    FlashAttention gradient from the FP4 forward's own output.
 *  - EFQ-Softmax abstract (AVQ Attention page; theflow "related" summary):
 *    the FlashAttention-style data flow with block-scaled E2M1 probabilities
 *    produced by the exp-then-quantize path, where one quantized P feeds both
 *    the PV numerator and the P.1 denominator, while the row-max update,
 *    historical rescaling, wide accumulation and final normalisation are
 *    those of FlashAttention.
 *  - HiFA4 abstract (theflow "related" page): QK^T and PV both run as 4-bit
 *    GEMMs with the online-softmax state kept wider (fp32 here).
 *
 * Number format (MXFP4, OCP Microscaling reading of "microscaling FP4"):
 *  - E2M1 code, 4 bits: bit 3 sign, magnitudes {0,.5,1,1.5,2,3,4,6} for
 *    codes 0..7; two codes per byte, element 2c in bits 3..0 and element
 *    2c+1 in bits 7..4.
 *  - E8M0 scale, 1 byte per 32 consecutive elements of the contraction
 *    axis: value 2^(byte-127); byte = clamp(floor(log2 amax) - 2, -127, 127)
 *    + 127 (amax < 2^-126 counts as 2^-127); 0xFF is never written.
 *  - element code = round-to-nearest-even of x / 2^(byte-127) onto the
 *    grid, ties to the even code, saturating at 6, sign kept (-0 -> 0x8).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors on ROCm), contiguous, row-major, 16-byte aligned.  The caller
 *    owns and allocates every buffer; the library never allocates, frees or
 *    synchronises, and keeps no state beyond two per-device caches: the arch
 *    check and the device address of the no-alloc entry point's array.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously on it; nothing is waited for.
 *  - Every function returns an attn_fp4_status; argument errors are
 *    detected on the host before anything is launched.  No exceptions cross
 *    the ABI, nothing is printed, nothing aborts.
 *  - Preconditions that are not checked: inputs finite; output buffers do
 *    not overlap inputs or each other.
 *  - Key-tile width: the forward visits keys in ascending tiles of 64 and
 *    quantizes P per row over the tile's two 32-key blocks against the
 *    running maximum after that tile; N must therefore be a multiple of 64.
 */
#ifndef ATTN_FP4_H
#define ATTN_FP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_FP4_OK = 0,
  ATTN_FP4_E_INVALID_ARG = 1,        /* null/misaligned pointer, bad shape, bad enum value */
  ATTN_FP4_E_UNSUPPORTED_DEVICE = 2, /* current device is not gfx950 */
  ATTN_FP4_E_UNSUPPORTED = 3,        /* valid request this build does not implement */
  ATTN_FP4_E_HIP = 4,                /* a HIP runtime call or kernel launch failed */
  ATTN_FP4_E_WORKSPACE = 5           /* workspace missing or smaller than required */
} attn_fp4_status;

/* Version of this ABI (structs and semantics); bumped on any change. */
int32_t attn_fp4_abi_version(void);

/* Static description of a status code (never NULL). */
const char* attn_fp4_status_string(int32_t status);

/*
 * attn_fp4_quantize -- bf16 -> MXFP4 (packed E2M1 codes + E8M0 scales).
 *
 * Follows the block-scaled E2M1 operand format of the EFQ-Softmax abstract
 * and the microscaling FP4 of the SageAttention3 title (Pengle Zhang page).
 *
 *   x       bf16 [bh, n, d], device.
 *   axis 0  quantize along d (Q and K): codes [bh, n, d/2] bytes,
 *           scales [bh, n, d/32] bytes.  Requires d % 32 == 0.
 *   axis 1  quantize along n (V), block-major: for each 32-token MX block b
 *           the 16 code bytes of every channel, then the next block --
 *           codes [bh, n/32, d, 16] (byte j of (b, c) holds tokens 32b+2j in
 *           the low and 32b+2j+1 in the high nibble), scales [bh, n/32, d].
 *           A 64-key tile of V^ is then one contiguous run of 32 d bytes.
 *           Requires n % 32 == 0 and d % 32 == 0.
 *   bh, n, d > 0.  Output is bit-exact with the rule in the header comment.
 * Errors: ATTN_FP4_E_INVALID_ARG for null or non-16-byte-aligned pointers,
 * non-positive sizes, a length not divisible as required, axis not 0/1.
 */
int32_t attn_fp4_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int32_t axis,
                          void* codes, void* scales, void* stream);

/*
 * Forward arguments.  Layouts (all device, contiguous):
 *   q_codes [B, Hq, N, d/2]   q_scales [B, Hq, N, d/32]   (attn_fp4_quantize axis 0)
 *   k_codes [B, Hkv, N, d/2]  k_scales [B, Hkv, N, d/32]  (axis 0)
 *   v_codes [B, Hkv, N/32, d, 16]  v_scales [B, Hkv, N/32, d]  (axis 1, block-major)
 *   o       bf16 [B, Hq, N, d]            (output, round-to-nearest-even)
 *   m       fp32 [B, Hq, N]  final row max of the scaled scores (natural-log
 *                            units, i.e. of s = scale * q.k)        (output)
 *   l       fp32 [B, Hq, N]  final row sum of the quantized P      (output)
 * Query head h reads KV head h / (Hq / Hkv).  causal != 0 masks keys j > i
 * (top-left aligned, equal query and key lengths).  softmax_scale <= 0
 * selects 1/sqrt(d).  Supported: d == 128 or d == 64, N % 64 == 0,
 * Hq % Hkv == 0.
 */
typedef struct {
  const void* q_codes;
  const void* q_scales;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  void* o;
  float* m;
  float* l;
  int64_t B, Hq, Hkv, N, d;
  int32_t causal;
  float softmax_scale;
  int32_t p_rule;     /* how P~ is formed, see ATTN_FP4_P_* */
} attn_fp4_fwd_args;

/*
 * P~ rules of the forward:
 *   ATTN_FP4_P_EXP  exp-then-quantize (the method's definition): P~ = MXFP4 of
 *                   p = exp(s - m) per 32-key block.
 *   ATTN_FP4_P_EFQ  exp-free codes after the EFQ-Softmax abstract, in this
 *                   library's reading (the pages give no formula): per block
 *                   the same E8M0 exponent e from the block maximum, then code
 *                   k = clamp(round_half_even(A y + B), 0, 7) of the residual
 *                   y = log2(p) - e computed from the shifted score without an
 *                   exponential; A = 1.7470566, B = 2.3141184 is the
 *                   least-squares line through (log2 v, k) of the seven
 *                   non-zero E2M1 magnitudes v.  attn_fp4_bwd_recompute
 *                   implements the exp rule only.
 */
enum { ATTN_FP4_P_EXP = 0, ATTN_FP4_P_EFQ = 1 };

/*
 * attn_fp4_fwd -- MXFP4 attention forward (Attn-QAT FP4 forward; EFQ-Softmax
 * exp-then-quantize data flow; HiFA4 4-bit QK^T and PV).  Both GEMMs run
 * on the scaled FP4 matrix cores; the running max, running sum and the
 * output accumulator are fp32.  Bitwise deterministic.
 * Errors: ATTN_FP4_E_INVALID_ARG (null/misaligned pointer, bad dims),
 * ATTN_FP4_E_UNSUPPORTED (N * d / 2 above 2^31 - 1: one head's codes exceed the
 * kernels' 32-bit buffer offsets), ATTN_FP4_E_UNSUPPORTED_DEVICE,
 * ATTN_FP4_E_HIP (launch failure).
 */
int32_t attn_fp4_fwd(const attn_fp4_fwd_args* args, void* stream);

/*
 * Cache forward arguments (FP4 attention for LLM inference, Attn-QAT
 * abstract: new query rows attend to keys and values that were quantized
 * once and are kept; chunked prefill and decode).
 *   q_codes   [B, Hq, Nq, d/2]   q_scales [B, Hq, Nq, d/32]  (axis 0)
 *   k_codes   [B, Hkv, Nk, d/2]  k_scales [B, Hkv, Nk, d/32] (axis 0)
 *   v_codes   [B, Hkv, Nk/32, d, 16]  v_scales [B, Hkv, Nk/32, d]
 *             (axis 1 over the cache's whole capacity Nk, block-major)
 *   seqlens_k int32 [B] device array, 4-byte aligned: valid cache length
 *             L_b of sequence b (values are clamped to [0, Nk]); NULL means
 *             L_b = Nk.
 *   o bf16 [B, Hq, Nq, d]; m, l fp32 [B, Hq, Nq] (outputs, as attn_fp4_fwd)
 * The Nq new rows are the last Nq positions of each sequence: their keys
 * and values are already in the cache, and new row i sits at position
 * L_b - Nq + i.  Keys j < L_b are visible; with causal != 0 only those with
 * j <= L_b - Nq + i (bottom-right alignment).  A row that sees no key
 * (L_b = 0, or causal with L_b - Nq + i < 0) gets O = 0, m = -inf, l = 0.
 * Cache memory past L_b is read only inside the last 64-key tile and never
 * changes the result, except that the scale of a V^ block that holds both
 * valid and later positions is the one stored (the cache quantized as a
 * whole).  Key tiles are visited in ascending order and P~ is requantized
 * per 32-key block exactly as in attn_fp4_fwd, so with Nq = Nk = L_b this is
 * attn_fp4_fwd.  p_rule as for attn_fp4_fwd.
 * Supported: d == 128 or d == 64, Nq >= 1, Nk % 64 == 0, Hq % Hkv == 0.
 * workspace: optional device memory (256-byte aligned) of at least
 * attn_fp4_fwd_kvcache_workspace_bytes(...) bytes.  When that size is not 0
 * (few query rows per KV head: decode, short chunks) and the workspace is
 * given, the key tiles are split over more workgroups: a first pass finds
 * each split's largest visible score, each split then starts from the
 * running max the sequential loop would carry into it (so every P~ code is
 * the one-pass code), and a last pass merges the splits; only the fp32
 * summation order of the output differs.  With workspace == NULL the
 * one-pass kernel runs.  Contents on entry do not matter; clobbered.
 * Errors: ATTN_FP4_E_INVALID_ARG (null/misaligned pointer, bad dims or
 * enum), ATTN_FP4_E_UNSUPPORTED (Nk * d / 2 above 2^31 - 1),
 * ATTN_FP4_E_WORKSPACE (given but too small or misaligned),
 * ATTN_FP4_E_UNSUPPORTED_DEVICE, ATTN_FP4_E_HIP.
 */
typedef struct {
  const void* q_codes;
  const void* q_scales;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  const int32_t* seqlens_k;
  void* o;
  float* m;
  float* l;
  void* workspace;
  int64_t workspace_bytes;
  int64_t B, Hq, Hkv, Nq, Nk, d;
  int32_t causal;
  float softmax_scale;
  int32_t p_rule;
} attn_fp4_fwd_kvcache_args;

/* Workspace bytes for the split cache forward of this shape: 0 when the
 * one-pass kernel is used anyway, -1 for an unsupported shape. */
int64_t attn_fp4_fwd_kvcache_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                             int64_t d);

int32_t attn_fp4_fwd_kvcache(const attn_fp4_fwd_kvcache_args* args, void* stream);

/*
 * attn_fp4_fwd_kvcache_noalloc -- attn_fp4_fwd_kvcache for callers that
 * cannot allocate device memory (code under HIP graph capture, tight decode
 * loops, harnesses that forbid hipMalloc).  Same arguments, layouts, results
 * and errors, except that args->workspace and args->workspace_bytes are
 * ignored: when the split path applies, its workspace is a device array inside
 * the library of ATTN_FP4_KVCACHE_SCRATCH_BYTES, one copy on every GPU the
 * library runs on, held until the process ends.  The call allocates and frees
 * nothing.  The array keeps the last call's contents; nothing in it needs to
 * start at zero.  All calls on one GPU share that GPU's array, so calls that
 * overlap on one GPU (concurrent streams, or threads) race: the caller orders
 * them, e.g. on one stream.  Its device address is looked up on the first
 * call on each device (with that device current).
 * Errors: as attn_fp4_fwd_kvcache; ATTN_FP4_E_WORKSPACE when the shape's split
 * workspace (attn_fp4_fwd_kvcache_workspace_bytes) exceeds
 * ATTN_FP4_KVCACHE_SCRATCH_BYTES (use attn_fp4_fwd_kvcache with a workspace).
 */
#define ATTN_FP4_KVCACHE_SCRATCH_BYTES (16 * 1024 * 1024)
int32_t attn_fp4_fwd_kvcache_noalloc(const attn_fp4_fwd_kvcache_args* args, void* stream);

/*
 * Backward arguments.  Quantized operands as for the forward; o, m, l are
 * the forward's outputs; do_ is bf16 [B, Hq, N, d].  Outputs dq bf16
 * [B, Hq, N, d], dk and dv bf16 [B, Hkv, N, d] (summed over the query heads
 * that share a KV head).  workspace: device memory of at least
 * attn_fp4_bwd_workspace_bytes(...) bytes, 256-byte aligned; its contents
 * on entry do not matter and are clobbered.
 */
typedef struct {
  const void* q_codes;
  const void* q_scales;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  const void* o;
  const void* do_;
  const float* m;
  const float* l;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;
  int64_t workspace_bytes;
  int64_t B, Hq, Hkv, N, d;
  int32_t causal;
  float softmax_scale;
} attn_fp4_bwd_args;

/* Workspace bytes attn_fp4_bwd_recompute needs for these sizes (< 0 on invalid sizes). */
int64_t attn_fp4_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d);

/*
 * attn_fp4_bwd_recompute -- Attn-QAT backward (abstract's two principles):
 * S is recomputed with the same FP4 QK^T as the forward; D = rowsum(dO*O)
 * uses the FP4 forward's output O (fp32); P = exp(S - m)/l; the dV operand
 * is the requantized P (MXFP4 of exp(S - m) per 32-key block, divided by
 * l); dQ, dK, dV come from bf16 matrix-core products with fp32
 * accumulation, gradients passing straight through the quantizers.
 * Errors: as attn_fp4_fwd, plus ATTN_FP4_E_WORKSPACE, and
 * ATTN_FP4_E_UNSUPPORTED when (Hq / Hkv) * N * d * 2 bytes (one KV head's
 * group of bf16 [N, d] tensors) exceeds 2^31 - 1, the reach of the kernels'
 * 32-bit buffer offsets.
 */
int32_t attn_fp4_bwd_recompute(const attn_fp4_bwd_args* args, void* stream);

/*
 * ---- NVFP4-style operands (a second scale format) ----
 *
 * The pages name NVFP4 as a 4-bit format (TetraJet-v2 abstract) and compare
 * it with MXFP4 and HiF4 (RFQ abstract; HiFA4 abstract) but do not define
 * it.  This library's reading is the published NVFP4 layout:
 *  - E2M1 codes as above (two per byte, same nibble order);
 *  - one unsigned FP8 E4M3 block scale byte per 16 consecutive elements of
 *    the contraction axis (4 exponent bits, bias 7, 3 mantissa bits,
 *    subnormals, largest 448 = 0x7E; 0x7F is never written);
 *  - one fp32 tensor scale G per tensor.
 * Every step is fp32 with round-to-nearest-even:
 *   G = max(amax / 2688, 2^-117) over the whole tensor (2688 = 6 * 448);
 *   per block s = amax_block / (6 G), S = E4M3(s), ties to the even mantissa,
 *   saturating at 448; code = E2M1(x / (S G)), ties to even, saturating at
 *   6, sign kept; a block with S = 0 gets sign-only codes.
 *   value = G * S * E2M1(code).
 */

/*
 * attn_fp4_nv_quantize -- bf16 -> NVFP4-style codes, E4M3 block scales and
 * the tensor scale (three launches on `stream`: clear, tensor amax, encode).
 *   x       bf16 [bh, n, d], device.
 *   axis 0  along d (Q, K): codes [bh, n, d/2], scales [bh, n, d/16].
 *   axis 1  along n (V), transposed: codes [bh, d, n/2] (byte j of channel
 *           c holds tokens 2j (low nibble) and 2j+1), scales [bh, d, n/16].
 *           Requires n % 16 == 0.
 *   tensor_scale  device float[2], 8-byte aligned (output): [0] = G, [1] =
 *           the tensor's amax.  Pass [0] to attn_fp4_nv_fwd.
 *   Requires d % 32 == 0, bh, n > 0.  Codes, scales and G are bit-exact with
 *   the rule above.
 * Errors: ATTN_FP4_E_INVALID_ARG (null or misaligned pointer, sizes, axis),
 * ATTN_FP4_E_UNSUPPORTED_DEVICE, ATTN_FP4_E_HIP.
 */
int32_t attn_fp4_nv_quantize(const void* x, int64_t bh, int64_t n, int64_t d, int32_t axis, void* codes,
                             void* scales, float* tensor_scale, void* stream);

/*
 * NVFP4-style forward arguments.  Layouts (device, contiguous):
 *   q_codes [B, Hq, N, d/2]  q_scales [B, Hq, N, d/16]    (attn_fp4_nv_quantize axis 0)
 *   k_codes [B, Hkv, N, d/2] k_scales [B, Hkv, N, d/16]   (axis 0)
 *   v_codes [B, Hkv, d, N/2] v_scales [B, Hkv, d, N/16]   (axis 1)
 *   *_tensor_scale  device float* to each operand's G (8-byte aligned)
 *   o, m, l as for attn_fp4_fwd (l is the row sum of the quantized P, in
 *   probability units).
 *   workspace: device memory, 256-byte aligned, of at least
 *   attn_fp4_nv_fwd_workspace_bytes(...) bytes (the operands dequantized to
 *   fp16); contents on entry do not matter and are clobbered.
 */
typedef struct {
  const void* q_codes;
  const void* q_scales;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  const float* q_tensor_scale;
  const float* k_tensor_scale;
  const float* v_tensor_scale;
  void* o;
  float* m;
  float* l;
  void* workspace;
  int64_t workspace_bytes;
  int64_t B, Hq, Hkv, N, d;
  int32_t causal;
  float softmax_scale;
} attn_fp4_nv_fwd_args;

/* Workspace bytes attn_fp4_nv_fwd needs for these sizes (< 0 on invalid sizes). */
int64_t attn_fp4_nv_fwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d);

/*
 * attn_fp4_nv_fwd -- the attention forward of attn_fp4_fwd (exp-then-quantize,
 * ascending 64-key tiles, one quantized P for numerator and denominator) over
 * NVFP4-style operands.  P is requantized per 16 keys in the same format with
 * the tensor scale of amax = 1: S = E4M3(max p * 448), P~ = E2M1(p * 2688 / S)
 * * S / 2688.  gfx950's block-scaled matrix core takes power-of-two scales per
 * 32 elements only, so both products run on the fp16 matrix core, where
 * E2M1 * E4M3 values (at most 6 significant bits, within 2^-10 .. 2688) are
 * exact; fp32 accumulation and softmax state; O is bf16.
 * Supported: d == 128 or d == 64, N % 64 == 0, Hq % Hkv == 0.
 * Errors: ATTN_FP4_E_INVALID_ARG, ATTN_FP4_E_WORKSPACE,
 * ATTN_FP4_E_UNSUPPORTED (N * d * 2 above 2^31 - 1: one head's fp16 operand
 * exceeds the kernel's 32-bit buffer offsets), ATTN_FP4_E_UNSUPPORTED_DEVICE,
 * ATTN_FP4_E_HIP.
 */
int32_t attn_fp4_nv_fwd(const attn_fp4_nv_fwd_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FP4_H */
