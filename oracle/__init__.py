"""CPU oracle for 4-bit (MXFP4) FlashAttention-style attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product path (the HIP library and its Python binding)
never imports, links or executes anything here, and this package imports
nothing from the product path.

Everything here is plain NumPy in float64 and deliberately slow: no
blocking, fusion or reordering beyond what the method itself prescribes, so
that each step can be checked by eye against the pages it follows:

* Attn-QAT: 4-Bit Attention With Quantization-Aware Training (abstract) --
  the method: FP4 forward, backward that recomputes the attention scores with
  the same low-precision QK^T, and the precision of the D term of the
  FlashAttention gradient.
* EFQ-Softmax abstract (the AVQ Attention page and the theflow "related"
  summary) -- the FlashAttention-style data flow with block-scaled E2M1
  probabilities: row-max update, historical rescaling, high-precision
  accumulation, final normalisation, and one quantized P used for both the
  PV numerator and the P.1 denominator.
* HiFA4 abstract (theflow "related" page) -- QK^T and PV both executed as
  4-bit GEMMs inside FlashAttention with the online-softmax state kept in a
  wider format.

* TetraJet-v2, RFQ and HiFA4 abstracts -- NVFP4 and HIF4 named as other
  4-bit formats; nv.py holds an NVFP4-style reading of that name.

Parity status of each function is stated in its module header.
"""

from .efq import EFQ_A, EFQ_B, efq_block_exponent, efq_codes, efq_fake_quant  # noqa: F401
from .mx import (  # noqa: F401
    E2M1_GRID,
    MX_BLOCK,
    decode_e2m1,
    e2m1_round_codes,
    mx_scale_exponent,
    quantize_mx,
    dequantize_mx,
    fake_quant_mx,
    pack_nibbles,
    unpack_nibbles,
)
from .nv import (  # noqa: F401
    E4M3_POS,
    NV_BLOCK,
    NV_TENSOR_DIV,
    decode_e4m3,
    e4m3_round_codes,
    nv_tensor_scale,
    quantize_nv,
    dequantize_nv,
    fake_quant_nv,
    nv_p_fake_quant,
)
from .attention import (  # noqa: F401
    BC,
    softmax_attention,
    attn_fwd,
    attn_fwd_kvcache,
    attn_bwd,
    attn_row_max,
)
