"""Write the oracle regression fixtures in this folder (tests/golden/*.txt).

Every stored value here is computed by ``oracle/`` alone, on inputs drawn by the seeded generator
(``bit_attention_amd.workloads``, which holds none of the method's arithmetic), and nothing here
comes from the HIP library.  The pages print no worked numeric example for any step of the path,
so these fixtures are not pins of the oracle against the pages: they record what the oracle
computes today, so that any later change to its arithmetic shows up in ``tests/test_golden.py``
and has to be made on purpose (regenerate with ``python tests/golden/make_golden.py``).

Fixture format: ``#`` lines are comments; every other line is ``key: value value ...`` with
integers in hex (``0x..``) or floats in Python's round-trip ``repr``.
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from bit_attention_amd import workloads  # noqa: E402

TINY = "tiny_b1h2n256d64"
FWD_ROWS = {0: (0, 65, 255), 1: (31, 128)}          # head -> sampled query rows
BWD_ROWS = (0, 100, 255)                            # dQ rows (head 0), dK / dV keys (head 1)


def _hex(a):
    return " ".join("0x%x" % int(x) for x in np.asarray(a).reshape(-1))


def _flt(a):
    return " ".join(repr(float(x)) for x in np.asarray(a, dtype=np.float64).reshape(-1))


def _write(name, header, items):
    path = os.path.join(HERE, name)
    with open(path, "w") as f:
        for line in header:
            f.write("# " + line + "\n")
        for key, val in items:
            f.write("%s: %s\n" % (key, val))
    return path


def tiny_inputs():
    return [workloads.gen_tensor(TINY, t) for t in ("q", "k", "v")]


def quantize_items():
    q, _, v = tiny_inputs()
    items = []
    # Q head (0, 0), rows 0..3, quantized along d: 64 codes and 2 scale bytes per row
    c, s = oracle.quantize_mx(q[0, 0, :4], axis=-1)
    for r in range(4):
        items += [("q_row%d_codes" % r, _hex(c[r])), ("q_row%d_scales" % r, _hex(s[r]))]
    # V head (0, 1), tokens 0..63 of channels 0..3, quantized along N: per channel 64 codes, 2 scales
    c, s = oracle.quantize_mx(v[0, 1, :64, :4], axis=0)
    for ch in range(4):
        items += [("v_ch%d_codes" % ch, _hex(c[:, ch])), ("v_ch%d_scales" % ch, _hex(s[:, ch]))]
    return items


def fwd_items():
    q, k, v = tiny_inputs()
    items = []
    for rule in ("exp", "efq"):
        for causal in (False, True):
            tag = "%s_%s" % (rule, "causal" if causal else "full")
            for h, rows in FWD_ROWS.items():
                o, m, l = oracle.attn_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], causal=causal,
                                          rows=np.array(rows), p_rule=rule)
                for i, r in enumerate(rows):
                    items += [("%s_h%d_r%d_m" % (tag, h, r), _flt(m[0, 0, i])),
                              ("%s_h%d_r%d_l" % (tag, h, r), _flt(l[0, 0, i])),
                              ("%s_h%d_r%d_o" % (tag, h, r), _flt(o[0, 0, i]))]
    return items


def bwd_items():
    q, k, v = tiny_inputs()
    do = workloads.gen_tensor(TINY, "do")
    items = []
    for causal in (False, True):
        tag = "causal" if causal else "full"
        o, m, l = oracle.attn_fwd(q, k, v, causal=causal)
        dq, dk, dv = oracle.attn_bwd(q, k, v, o, do, m, l, causal=causal)
        for r in BWD_ROWS:
            items += [("%s_dq_h0_r%d" % (tag, r), _flt(dq[0, 0, r])),
                      ("%s_dk_h1_k%d" % (tag, r), _flt(dk[0, 1, r])),
                      ("%s_dv_h1_k%d" % (tag, r), _flt(dv[0, 1, r]))]
    return items


FIXTURES = {
    "mx_quantize_tiny.txt": (
        ["MXFP4 quantization (E2M1 codes, one E8M0 scale byte per 32 elements) by oracle.quantize_mx:",
         "Q along d (head dim) and V along N (sequence), as the Attn-QAT and EFQ-Softmax abstracts",
         "quantize the operands of QK^T and PV.  Inputs: workload %s, seeded generator." % TINY,
         "Codes are unpacked (one 4-bit code per value, sign in bit 3); scales are biased exponents."],
        quantize_items),
    "attn_fwd_tiny.txt": (
        ["Attention forward by oracle.attn_fwd on workload %s (B1 H2 N256 d64):" % TINY,
         "64-key tiles, running max, P~ = MXFP4(exp(s - m)) per 32-key block ('exp', the definition)",
         "or the EFQ reading of the exp-free codes ('efq'); non-causal ('full') and causal.",
         "Per sampled row: m (natural-log units, scaled scores), l (sum of P~) and O (64 values)."],
        fwd_items),
    "attn_bwd_tiny.txt": (
        ["Straight-through backward by oracle.attn_bwd (FP4 recomputation of the scores, P~ / l in dV,",
         "the unquantized P in dS; Attn-QAT abstract) on workload %s with dO from the generator," % TINY,
         "from the oracle's own forward outputs.  dQ rows of head 0, dK and dV key rows of head 1."],
        bwd_items),
}


def main():
    for name, (header, fn) in FIXTURES.items():
        print("wrote", _write(name, header + ["Generated by tests/golden/make_golden.py (oracle/ only)."], fn()))


if __name__ == "__main__":
    main()
