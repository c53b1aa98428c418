"""MXFP4 (4-bit) FlashAttention forward and Attn-QAT backward for MI355X (gfx950).

The compute lives in ``libattnfp4.so`` (hand-written HIP, C ABI declared in
``include/attn_fp4.h``).  ``bit_attention_amd.ops`` is a thin ctypes binding
with the same entry-point names; it only marshals arguments (torch tensors in
device memory, the current HIP stream) and raises if the library is missing.
``bit_attention_amd.workloads`` draws the seeded synthetic inputs.
"""
