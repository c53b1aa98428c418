"""GPU parity of attn_fp4_quantize: codes and scales bit-exact against the oracle."""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import to_dev

pytestmark = pytest.mark.gpu


def ref_quant(x, axis):
    """Oracle codes/scales in the library's layouts: axis 1 is block-major, [.., n/32, d, 16] codes
    (the 16 bytes of one channel's 32-token block) and [.., n/32, d] scales."""
    x = np.asarray(x, dtype=np.float64)
    if axis == 0:
        c, s = oracle.quantize_mx(x, axis=-1)
        return oracle.pack_nibbles(c, -1), s
    c, s = oracle.quantize_mx(np.swapaxes(x, -1, -2), axis=-1)      # per channel, along n
    packed = oracle.pack_nibbles(c, -1)                              # [.., d, n/2]
    d, n2 = packed.shape[-2:]
    blocks = packed.reshape(packed.shape[:-1] + (n2 // 16, 16))     # [.., d, n/32, 16]
    return np.ascontiguousarray(np.swapaxes(blocks, -3, -2)), np.ascontiguousarray(np.swapaxes(s, -1, -2))


def gpu_quant(x, axis):
    import torch
    from bit_attention_amd import ops
    c, s = ops.attn_fp4_quantize(to_dev(x, torch.bfloat16), axis)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def check(x, axis, label):
    gc, gs = gpu_quant(x, axis)
    rc, rs = ref_quant(x, axis)
    assert np.array_equal(gs, rs), "%s: scales differ at %d places" % (label, int((gs != rs).sum()))
    assert np.array_equal(gc, rc), "%s: codes differ at %d bytes" % (label, int((gc != rc).sum()))


def all_finite_bf16():
    u = np.arange(1 << 16, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("axis", [0, 1])
def test_exhaustive_bf16_sorted_and_shuffled(axis):
    x = all_finite_bf16()
    x = np.concatenate([x, np.zeros(65536 - x.size, dtype=np.float32)])   # pad to 1024 x 64
    # sorted by magnitude -> the 32 elements of a block share a binade, so every code region is hit
    srt = x[np.argsort(np.abs(x), kind="stable")]
    shuf = np.random.default_rng(3).permutation(x)
    for name, arr in (("sorted", srt), ("shuffled", shuf)):
        if axis == 0:
            blocks = arr.reshape(1, 1024, 64)            # blocks run along the last axis
        else:
            blocks = np.ascontiguousarray(arr.reshape(1, 64, 1024).transpose(0, 2, 1))  # along n
        check(blocks, axis, "exhaustive %s axis %d" % (name, axis))


@pytest.mark.parametrize("axis", [0, 1])
def test_special_values(axis):
    x = np.zeros((2, 64, 64), dtype=np.float32)
    x[0, :, 0] = -0.0
    x[0, 1, :] = 2.0 ** -133                  # smallest bf16 subnormal everywhere in a row
    x[0, 2, 5] = 3.3895313892515355e38        # largest finite bf16
    x[0, 2, 6] = -1.0
    x[0, 3, :] = np.where(np.arange(64) % 2, 6.0, -0.25)
    x[1] = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.96875], dtype=np.float32), (64, 8))
    check(x, axis, "special axis %d" % axis)


@pytest.mark.parametrize("shape,axis", [((3, 7, 96), 0), ((1, 1, 32), 0), ((2, 96, 160), 1), ((1, 32, 32), 1),
                                        ((5, 288, 64), 1)])
def test_ragged_shapes(shape, axis):
    rng = np.random.default_rng(sum(shape) + axis)
    x = W.round_to_bf16(rng.standard_t(3, size=shape) * 3)
    check(x, axis, "ragged %s axis %d" % (shape, axis))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_tensors_full_launch_sampled_heads(name):
    """Quantize each workload tensor whole (the launch the bench times); compare sampled heads."""
    import torch
    from bit_attention_amd import ops
    w = W.WORKLOADS[name]
    tensors = [("q", 0), ("k", 0), ("v", 1)] + ([("do", 0)] if w.backward else [])
    for t, axis in tensors:
        x = W.gen_tensor(w, t)
        c, s = ops.attn_fp4_quantize(to_dev(x, torch.bfloat16), axis)
        torch.cuda.synchronize()
        c, s = c.cpu().numpy(), s.cpu().numpy()
        H = x.shape[1]
        heads = sorted({(0, 0), (w.B - 1, H - 1), (w.B // 2, H // 2)})
        for b, h in heads:
            rc, rs = ref_quant(x[b, h], axis)
            assert np.array_equal(s[b, h], rs), (name, t, b, h)
            assert np.array_equal(c[b, h], rc), (name, t, b, h)
