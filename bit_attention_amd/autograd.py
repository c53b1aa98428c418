"""Attn-QAT training surface: FP4 attention as a torch.autograd.Function.

The forward quantizes Q, K (along d) and V (along the sequence) to MXFP4 and runs the fused FP4
attention forward; it keeps only the FP4 operands, O and the row statistics m, l for the
backward (about a quarter of the memory of keeping bf16 Q, K, V).  The backward is
attn_fp4_bwd_recompute: S is recomputed with the same FP4 QK^T and gradients pass straight
through the four quantizers (Attn-QAT abstract, principles (1) and (2)).  Every step runs in the
library's kernels; this module only marshals arguments.
"""

import torch

from . import ops


class FP4Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal=False, softmax_scale=0.0):
        qc, qs = ops.attn_fp4_quantize(q, 0)
        kc, ks = ops.attn_fp4_quantize(k, 0)
        vc, vs = ops.attn_fp4_quantize(v, 1)
        o, m, l = ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=causal, softmax_scale=softmax_scale)
        ctx.save_for_backward(qc, qs, kc, ks, vc, vs, o, m, l)
        ctx.causal = bool(causal)
        ctx.softmax_scale = float(softmax_scale)
        return o

    @staticmethod
    def backward(ctx, do):
        qc, qs, kc, ks, vc, vs, o, m, l = ctx.saved_tensors
        do = do.to(torch.bfloat16).contiguous()
        dq, dk, dv = ops.attn_fp4_bwd_recompute(qc, qs, kc, ks, vc, vs, o, do, m, l, causal=ctx.causal,
                                                softmax_scale=ctx.softmax_scale)
        return dq, dk, dv, None, None


def fp4_attention(q, k, v, causal=False, softmax_scale=0.0):
    """MXFP4 attention with the Attn-QAT backward.

    q [B, Hq, N, d], k and v [B, Hkv, N, d]: contiguous bf16 tensors on the GPU; d in {64, 128},
    N % 64 == 0, Hq % Hkv == 0.  softmax_scale <= 0 selects 1/sqrt(d).  Returns O bf16 [B, Hq, N, d].
    """
    return FP4Attention.apply(q, k, v, causal, softmax_scale)
