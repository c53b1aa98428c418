"""The HIP path against the stored oracle fixtures of tests/golden (written by make_golden.py from
the oracle alone).  Quantized codes and scale bytes must be identical; the forward's sampled rows
are held to the forward parity bar (rel-L2 <= 5e-3, max-abs <= 3e-2 plus the bf16 half-ulp on O,
m to 1e-5, l element-wise to 1e-4 relative)."""

import numpy as np
import pytest

from bit_attention_amd import workloads as W
from golden_io import generator_module, read_fixture
from helpers import compare, compare_l, to_dev

pytestmark = pytest.mark.gpu

MG = generator_module()


def _tiny():
    return [W.gen_tensor(MG.TINY, t) for t in ("q", "k", "v")]


def _unpack(packed):
    """Bytes holding two 4-bit codes each (low nibble first) -> one code per element."""
    p = np.asarray(packed, dtype=np.int64)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (-1,))


def test_quantize_matches_stored_codes():
    import torch
    from bit_attention_amd import ops
    q, _, v = _tiny()
    qc, qs = ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0)
    vc, vs = ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1)
    torch.cuda.synchronize()
    qc, qs, vc, vs = (t.cpu().numpy() for t in (qc, qs, vc, vs))
    g = read_fixture("mx_quantize_tiny.txt")
    for r in range(4):
        assert np.array_equal(_unpack(qc[0, 0, r]), g["q_row%d_codes" % r]), "Q row %d codes" % r
        assert np.array_equal(qs[0, 0, r].astype(np.int64), g["q_row%d_scales" % r]), "Q row %d scales" % r
    # V: block-major [.., N/32, d, 16] codes (one channel's 32-token block) and [.., N/32, d] scales
    for ch in range(4):
        codes = np.concatenate([_unpack(vc[0, 1, blk, ch]) for blk in range(2)])
        assert np.array_equal(codes, g["v_ch%d_codes" % ch]), "V channel %d codes" % ch
        assert np.array_equal(vs[0, 1, :2, ch].astype(np.int64), g["v_ch%d_scales" % ch]), "V ch %d scales" % ch


@pytest.mark.parametrize("rule", ["exp", "efq"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_stored_rows(rule, causal):
    import torch
    from bit_attention_amd import ops
    q, k, v = _tiny()
    dq = [to_dev(t, torch.bfloat16) for t in (q, k, v)]
    qc, qs = ops.attn_fp4_quantize(dq[0], 0)
    kc, ks = ops.attn_fp4_quantize(dq[1], 0)
    vc, vs = ops.attn_fp4_quantize(dq[2], 1)
    o, m, l = ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=causal,
                               p_rule=ops.P_EFQ if rule == "efq" else ops.P_EXP)
    torch.cuda.synchronize()
    o, m, l = o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    g = read_fixture("attn_fwd_tiny.txt")
    tag = "%s_%s" % (rule, "causal" if causal else "full")
    for h, rows in MG.FWD_ROWS.items():
        rows = list(rows)
        ro = np.stack([g["%s_h%d_r%d_o" % (tag, h, r)] for r in rows])
        rm = np.array([g["%s_h%d_r%d_m" % (tag, h, r)][0] for r in rows])
        rl = np.array([g["%s_h%d_r%d_l" % (tag, h, r)][0] for r in rows])
        compare(o[0, h, rows], ro, "%s head %d O" % (tag, h))
        assert np.max(np.abs(m[0, h, rows] - rm)) <= 1e-5 * max(1.0, np.abs(rm).max()), tag
        compare_l(l[0, h, rows], rl, "%s head %d l" % (tag, h))
