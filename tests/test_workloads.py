"""Seeded synthetic inputs: determinism, per-head independence and the stated distributions."""

import numpy as np

from bit_attention_amd.workloads import WORKLOADS, gen_head, gen_tensor, round_to_bf16, sample_rows


def test_bf16_rounding_is_rne_and_exact_on_bf16():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -7], dtype=np.float64)
    r = round_to_bf16(x)
    assert r.tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 1.0 + 2.0 ** -7]
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_heads_are_deterministic_and_independent():
    w = WORKLOADS["tiny_b1h2n256d64"]
    a = gen_tensor(w, "q")
    assert np.array_equal(a[0, 1], gen_head(w, "q", 0, 1))
    assert not np.array_equal(a[0, 0], a[0, 1])
    assert not np.array_equal(gen_head(w, "q", 0, 0), gen_head(w, "k", 0, 0))
    assert a.dtype == np.float32 and a.shape == (1, 2, 256, 64)


def test_llm_outlier_channels_shared_by_q_and_k():
    w = WORKLOADS["llm_causal_b2h16n4096d128"]
    q = gen_head(w, "q", 1, 3)
    k = gen_head(w, "k", 1, 3)
    cq = np.argsort(q.std(0))[-2:]
    ck = np.argsort(k.std(0))[-2:]
    assert set(cq) == set(ck)
    assert np.all(q.std(0)[cq] > 10)
    v = gen_head(w, "v", 1, 3)
    assert np.abs(v).max() > 20          # Student-t(3) tails


def test_gqa_k_outlier_and_dit_heavy_tails():
    w = WORKLOADS["gqa_causal_b1hq32hkv8n16384d128"]
    k = gen_head(w, "k", 0, 2)
    s = np.sort(k.std(0))
    assert s[-1] > 20 and s[-2] < 1.2
    w = WORKLOADS["dit_b1h24n32768d128"]
    x = gen_head(w, "v", 0, 0).astype(np.float64)
    assert 0.8 < x.std() / np.exp(0.25) ** 1 < 1.6   # t(4)/sqrt(2) * lognormal(0, 0.5)


def test_sample_rows():
    r = sample_rows(32768, 512)
    assert r.shape == (512,) and np.all(np.diff(r) > 0)
    assert r[0] == 0 and r[-1] == 32767 and 63 in r and 32704 in r
    assert np.array_equal(sample_rows(256, 512), np.arange(256))
